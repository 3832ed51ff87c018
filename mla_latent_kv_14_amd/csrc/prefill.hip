// The decompressed branch (bhfrc.com/news/60867 S1, S3, S6: prefill takes the decompressing
// path and decode the absorbed one, split at a threshold on the number of query rows). With T
// query tokens per sequence at or above the threshold, the per-head keys and values are
// expanded once per cached token, and attention runs at the head widths instead of the latent
// width:
//   K_nope[t,h,:] = W_UK[h] c_KV[t]            (d_nope values; lpnh.cn/news/2494972 S2.1)
//   V[t,h,:]      = W_UV[h]^T c_KV[t]          (d_v values)
//   s(i,t,h)      = scale (q_nope[i,h] . K_nope[t,h] + q_rope[i,h] . k_R[t])
//   out[i,h,:]    = sum_t softmax_t(s) V[t,h,:]  over t <= S_b - T + i (causal)
// which is the absorbed decode's result up to rounding (the two differ only in where W_UK and
// W_UV are applied).
//
// Kernels:
//   transpose: W_UVt[h][e][c] = W_UV[h][c][e], so that both weights are read along the latent
//     (contraction) dimension.
//   decompress: per (sequence, 256 tokens, head, K or V): out^T[128 columns x 256 tokens] =
//     W (columns x d_c) . c_KV^T with W = W_UK[h] or W_UVt[h], 32x32x16 bf16 MFMA over d_c in
//     chunks of 32 staged in LDS (two chunks in flight in registers; two work groups per CU),
//     rows of the page-table-addressed cache gathered directly; bf16 out into the workspace,
//     [sequence][head][token][width], so that a work group's block is contiguous.
//   attention: per (sequence, head, 128 query rows): four waves of 32 rows share each 32-token
//     tile of [K_nope | k_R] and V in LDS (k_R straight from the paged cache), S^T = K Q^T and
//     O^T += V^T P^T on 32x32x16 MFMA (the contraction index of P numbered in the order the
//     score layout holds tokens), online softmax per row in the log2 domain.
#include <type_traits>

#include "device.h"
#include "kernels.h"

namespace mla {

namespace pf {
constexpr int NT = 256;       // threads per work group (four waves)
constexpr int DTOK = 256;     // decompress: tokens per work group
constexpr int DCOL = 128;     // decompress: output columns per work group (one head's K or V)
constexpr int DKC = 32;       // decompress: contraction chunk
constexpr int DNT = 512;      // decompress: threads per work group (eight waves)
constexpr int QB = 128;       // attention: query rows per work group (32 per wave)
constexpr int TT = 32;        // attention: tokens per tile
}  // namespace pf

// 16-byte chunk c of row r inside a row of `nch` chunks, XOR-swizzled within groups of 8 (or
// of the row when shorter) by the row, so that reads of one chunk column across rows spread
// over the banks.
template <int NCH>
__device__ __forceinline__ int pf_chunk(int r, int c) {
  constexpr int G = NCH < 8 ? NCH : 8;
  return (c & ~(G - 1)) | ((c & (G - 1)) ^ ((r >> 1) & (G - 1)));
}

// ---------------------------------------------------------------- W_UV transpose
template <int DC, int DV>
__global__ void __launch_bounds__(256) transpose_wuv_kernel(const uint16_t* __restrict__ W_UV,
                                                            uint16_t* __restrict__ W_UVt) {
  __shared__ uint16_t t[32][33];
  const int h = blockIdx.z, c0 = blockIdx.y * 32, e0 = blockIdx.x * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
  const uint16_t* src = W_UV + (size_t)h * DC * DV;
  uint16_t* dst = W_UVt + (size_t)h * DV * DC;
#pragma unroll
  for (int k = 0; k < 4; ++k) t[ty + 8 * k][tx] = src[(size_t)(c0 + ty + 8 * k) * DV + e0 + tx];
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 4; ++k) dst[(size_t)(e0 + ty + 8 * k) * DC + c0 + tx] = t[tx][ty + 8 * k];
}

// ---------------------------------------------------------------- decompression
// 16-byte chunk c of LDS row r of the decompression's 64-byte rows, XOR-swizzled by r / 4: 16
// consecutive rows read at one chunk column then cover all 16 chunk slots of a 256-byte span
// of the banks.
__device__ __forceinline__ int dc_chunk(int r, int c) { return c ^ ((r >> 2) & 3); }

// Per group of sequences: out[t][n] = sum_c c_KV[t][c] * W[n][c] for the keys (W = W_UK[h],
// n < DN) and the values (W = W_UVt[h], n < DV) of every head. A work group computes one
// half (K or V) of one head for 256 tokens; the grid puts the halves of all heads first, so
// that the work groups in flight share their token tile (the gathered cache rows come from
// L2). Eight waves, each a 64 x 64 block of the output (columns 64 (wave & 1), tokens
// 64 (wave >> 1)) as 2 x 2 MFMA 32x32x16 blocks. The contraction runs in chunks of 32 staged in
// LDS (two buffers) with the next two chunks' global loads in flight in registers. At 64
// accumulator registers the kernel fits in 128 per lane, so two work groups share a CU and
// one's output stores overlap the other's MFMAs.
// Grid: x = 2 * head + half, y = 256-token block of the sequence, z = sequence of the group.
template <int H, int DN, int DC, int DR, int DV>
__global__ void __launch_bounds__(pf::DNT, 2)
decompress_kernel(const char* __restrict__ kv, const int32_t* __restrict__ page_table,
                  const int32_t* __restrict__ seq_lens, int b0, int max_pages, int num_pages,
                  const uint16_t* __restrict__ W_UK, const uint16_t* __restrict__ W_UVt,
                  uint16_t* __restrict__ kbuf, uint16_t* __restrict__ vbuf, int smax) {
  using namespace pf;
  constexpr int ROWB = (DC + DR) * 2;   // bytes per cache token row
  constexpr int NCH = DKC * 2 / 16;     // 16-byte chunks per LDS row (4)
  constexpr int PA = DTOK * NCH / DNT;  // 16-byte cache-row pieces per thread per chunk (2)
  constexpr int NCHUNK = DC / DKC;
  constexpr int DEPTH = NCHUNK > 2 ? 2 : 1;  // chunks in flight in registers
  static_assert(DC % DKC == 0 && DN <= DCOL && DV == DCOL, "shape");
  static_assert(DTOK == 256 && DCOL == 128 && DKC == 32 && PA == 2 && DNT == 512,
                "piece mapping");
  // LDS: the two chunk buffers [W rows | cache rows], then (after the contraction) each wave's
  // 64 x 64 output block, staged so that it leaves as whole 128-byte rows
  constexpr int WB = DCOL * DKC * 2, AB = DTOK * DKC * 2;  // bytes of one buffer's parts
  constexpr int STG = 64 * 128;                             // bytes of one wave's block
  constexpr int LDS_BYTES = 2 * (WB + AB) > 8 * STG ? 2 * (WB + AB) : 8 * STG;
  __shared__ __attribute__((aligned(16))) char lds[LDS_BYTES];
  auto lds_w = [&](int buf) { return (MLA_LDS char*)lds + buf * WB; };
  auto lds_a = [&](int buf) { return (MLA_LDS char*)lds + 2 * WB + buf * AB; };
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = blockIdx.x >> 1, part = blockIdx.x & 1, sl = blockIdx.z, b = b0 + sl;
  const int t0 = blockIdx.y * DTOK;
  // S_b within the page table and within the rows the workspace keeps per sequence (smax,
  // the dims' max_seq_len: S_b <= max_seq_len is the caller's contract, enforced here)
  const int S = min(clamp_len(seq_lens[b], max_pages), smax);
  if (t0 >= S) return;
  const int width = part == 0 ? DN : DV;

  // thread tid moves 16-byte chunk c = tid % 4 of weight row tid / 4 and of cache rows
  // tid / 4 + 128k (k < 2)
  const int c = tid & 3, rb = tid >> 2;
  const bool wok = rb < width;  // K rows past DN are zero
  const uint16_t* wsrc = (part == 0 ? W_UK + ((size_t)h * DN + (wok ? rb : 0)) * DC
                                    : W_UVt + ((size_t)h * DV + rb) * DC) + 8 * c;
  const uint32_t wlo = (uint32_t)(rb * DKC * 2 + 16 * dc_chunk(rb, c));
  const char* asrc[PA];
  uint32_t alo[PA];
#pragma unroll
  for (int k = 0; k < PA; ++k) {
    const int r = rb + 128 * k;
    const int t = min(t0 + r, S - 1);  // rows past the end repeat the last token (unused)
    int page = page_table[(size_t)b * max_pages + t / kPage];
    page = page < 0 ? 0 : (page >= num_pages ? num_pages - 1 : page);
    asrc[k] = kv + ((size_t)page * kPage + t % kPage) * ROWB + 16 * c;
    alo[k] = (uint32_t)(r * DKC * 2 + 16 * dc_chunk(r, c));
  }
  u32x4 wreg[DEPTH], areg[DEPTH][PA];
  auto load_chunk = [&](int kc, int slot) {
    wreg[slot] = wok ? *reinterpret_cast<const u32x4*>(wsrc + kc * DKC) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int k = 0; k < PA; ++k)
      areg[slot][k] = *reinterpret_cast<const u32x4*>(asrc[k] + kc * DKC * 2);
  };
  auto store_chunk = [&](int slot, int buf) {
    *reinterpret_cast<MLA_LDS u32x4*>(lds_w(buf) + wlo) = wreg[slot];
#pragma unroll
    for (int k = 0; k < PA; ++k)
      *reinterpret_cast<MLA_LDS u32x4*>(lds_a(buf) + alo[k]) = areg[slot][k];
  };

  const int mw = 64 * (wave & 1), nw = 64 * (wave >> 1);
  const int r32 = lane & 31, hi = lane >> 5;
  f32x16 acc[2][2] = {};
#pragma unroll
  for (int kc = 0; kc < DEPTH; ++kc) load_chunk(kc, kc);
  store_chunk(0, 0);
  if (DEPTH < NCHUNK) load_chunk(DEPTH, 0);
  __syncthreads();
#pragma unroll
  for (int kc = 0; kc < NCHUNK; ++kc) {
    const int buf = kc & 1;
    const MLA_LDS char* wl = lds_w(buf);
    const MLA_LDS char* al = lds_a(buf);
#pragma unroll
    for (int ks = 0; ks < DKC / 16; ++ks) {
      bf16x8 wa[2], ab[2];
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int r = mw + 32 * m + r32;
        wa[m] = lds_read_b128(wl, r * DKC * 2 + 16 * dc_chunk(r, 2 * ks + hi));
      }
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        const int r = nw + 32 * n + r32;
        ab[n] = lds_read_b128(al, r * DKC * 2 + 16 * dc_chunk(r, 2 * ks + hi));
      }
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int n = 0; n < 2; ++n) acc[m][n] = mfma_32x32x16(wa[m], ab[n], acc[m][n]);
    }
    if (kc + 1 < NCHUNK) {
      // chunk kc+1 (loaded DEPTH - 1 chunks ago) into the other buffer, whose last reads were
      // before the last barrier; then its register slot takes chunk kc+1+DEPTH
      store_chunk((kc + 1) % DEPTH, buf ^ 1);
      if (kc + 1 + DEPTH < NCHUNK) load_chunk(kc + 1 + DEPTH, (kc + 1) % DEPTH);
      __syncthreads();
    }
  }
  // out^T block (m, n): lane holds token nw + 32n + r32 and columns mw + 32m + 8(i/4) + 4hi +
  // i%4 (i < 16). The wave's 64 x 64 block is staged in LDS (row = token, 16-byte chunk
  // 4m + g of the row XOR-swizzled by row % 8) and read back as whole 128-byte rows, eight
  // lanes per row: a store then covers whole lines instead of 16 bytes of 32 lines. Output
  // layout [sequence][head][token][width]; K columns at or past DN (the zero rows) and tokens
  // past S are not stored.
  __syncthreads();  // every wave is done with the chunk buffers
  MLA_LDS char* const stg = (MLA_LDS char*)lds + wave * STG;
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const int row = 32 * n + r32;
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x16& o = acc[m][n];
        const u32x2 w = {pack_bf16x2(o[4 * g], o[4 * g + 1]),
                         pack_bf16x2(o[4 * g + 2], o[4 * g + 3])};
        *reinterpret_cast<MLA_LDS u32x2*>(stg + row * 128 + 16 * ((4 * m + g) ^ (row & 7)) +
                                          8 * hi) = w;
      }
  }
  uint16_t* const dst = (part == 0 ? kbuf : vbuf) + ((size_t)sl * H + h) * smax * width;
  const int cl = lane & 7;  // 16-byte chunk of the row: columns mw + 8cl .. +8
  // Written non-temporally: the attention kernel reads each row once, later, and streaming
  // stores leave the cache to the latent tiles still being decompressed.
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = 8 * i + (lane >> 3);
    const int t = t0 + nw + row;
    const u32x4 v = *reinterpret_cast<const MLA_LDS u32x4*>(stg + row * 128 + 16 * (cl ^ (row & 7)));
    if (t < S && mw + 8 * cl + 8 <= width)
      __builtin_nontemporal_store(v,
                                  reinterpret_cast<u32x4*>(dst + (size_t)t * width + mw + 8 * cl));
  }
}

// ---------------------------------------------------------------- attention
// Grid: x = 128-row query block, y = head, z = sequence of the group.
template <int H, int DN, int DC, int DR, int DV>
__global__ void __launch_bounds__(pf::NT)
prefill_attn_kernel(const uint16_t* __restrict__ q_nope, const uint16_t* __restrict__ q_rope,
                    const char* __restrict__ kv, const int32_t* __restrict__ page_table,
                    const int32_t* __restrict__ seq_lens, int b0, int max_pages, int num_pages,
                    int T, const uint16_t* __restrict__ kbuf, const uint16_t* __restrict__ vbuf,
                    int smax, float scale_log2, uint16_t* __restrict__ out,
                    float* __restrict__ lse_out) {
  using namespace pf;
  constexpr int DK = DN + DR;             // score contraction width
  constexpr int KS = DK / 16;             // 32x32x16 steps over it
  constexpr int KCH = DK * 2 / 16;        // 16-byte chunks of a K row in LDS
  constexpr int NCH_N = DN * 2 / 16;      // of which from K_nope
  constexpr int VCH = DV * 2 / 16;        // 16-byte chunks of a V row
  constexpr int ROWB = (DC + DR) * 2;     // bytes per cache token row
  constexpr int PIECES = TT * (KCH + VCH);
  constexpr int PPT = PIECES / NT;        // 16-byte pieces per thread per tile
  static_assert(DK % 16 == 0 && DN % 8 == 0 && DR % 8 == 0 && KCH % 8 == 0 && VCH % 8 == 0 &&
                PIECES % NT == 0 && DV % 32 == 0, "shape");
  __shared__ __attribute__((aligned(16))) char lds_k[2][TT * DK * 2];
  __shared__ __attribute__((aligned(16))) char lds_v[2][TT * DV * 2];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int sl = blockIdx.z, b = b0 + sl, h = blockIdx.y;
  const int S = min(clamp_len(seq_lens[b], max_pages), smax);  // as in the decompression
  const int i0 = blockIdx.x * QB;  // first query row of the block
  // the block's last row sits at position S - T + min(T - 1, i0 + QB - 1): tokens past it are
  // masked for every row of the block
  const int last = S - T + min(T - 1, i0 + QB - 1);
  const int ntok = last + 1 > 0 ? last + 1 : 0;
  const int ntiles = (ntok + TT - 1) / TT;

  const int r32 = lane & 31, hi = lane >> 5;
  const int G16 = lane >> 4, q16 = lane & 15;
  const int qi = i0 + 32 * wave + r32;        // this lane's query row
  const int qc = qi < T ? qi : T - 1;         // (rows past T load a valid row, write nothing)
  const int pos = S - T + qi;                 // its position: attends to tokens 0 .. pos
  // query operand: B of S^T = K Q^T, lane = row r32, dims 16s + 8hi .. +8
  bf16x8 qf[KS];
  {
    const uint16_t* qn = q_nope + (((size_t)b * T + qc) * H + h) * DN;
    const uint16_t* qr = q_rope + (((size_t)b * T + qc) * H + h) * DR;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int d = 16 * s + 8 * hi;
      qf[s] = d < DN ? *reinterpret_cast<const bf16x8*>(qn + d)
                     : *reinterpret_cast<const bf16x8*>(qr + (d - DN));
    }
  }

  // tile loads: piece p = (token r, chunk c) of K (c < KCH: K_nope, then k_R) or V
  u32x4 reg[PPT];
  auto load_tile = [&](int j) {
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
      const int p = tid + NT * k;
      const int isv = p >= TT * KCH;
      const int q = isv ? p - TT * KCH : p;
      const int nch = isv ? VCH : KCH;
      const int r = q / nch, c = q - r * nch;
      int t = TT * j + r;
      t = t < S ? t : (S > 0 ? S - 1 : 0);  // past the end: a valid row, masked
      const uint16_t* src;
      if (isv) {
        src = vbuf + (((size_t)sl * H + h) * smax + t) * DV + 8 * c;
      } else if (c < NCH_N) {
        src = kbuf + (((size_t)sl * H + h) * smax + t) * DN + 8 * c;
      } else {
        int page = page_table[(size_t)b * max_pages + t / kPage];
        page = page < 0 ? 0 : (page >= num_pages ? num_pages - 1 : page);
        src = reinterpret_cast<const uint16_t*>(kv + ((size_t)page * kPage + t % kPage) * ROWB +
                                                DC * 2) + 8 * (c - NCH_N);
      }
      reg[k] = *reinterpret_cast<const u32x4*>(src);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
      const int p = tid + NT * k;
      const int isv = p >= TT * KCH;
      const int q = isv ? p - TT * KCH : p;
      const int nch = isv ? VCH : KCH;
      const int r = q / nch, c = q - r * nch;
      MLA_LDS char* base = isv ? (MLA_LDS char*)lds_v[buf] : (MLA_LDS char*)lds_k[buf];
      const int off = isv ? r * DV * 2 + 16 * pf_chunk<VCH>(r, c)
                          : r * DK * 2 + 16 * pf_chunk<KCH>(r, c);
      *reinterpret_cast<MLA_LDS u32x4*>(base + off) = reg[k];
    }
  };

  f32x16 acc[DV / 32] = {};
  float m_run = -INFINITY, l_lane = 0.f;
  if (ntiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();
  for (int j = 0; j < ntiles; ++j) {
    const int buf = j & 1;
    if (j + 1 < ntiles) load_tile(j + 1);
    const MLA_LDS char* kl = (const MLA_LDS char*)lds_k[buf];
    const MLA_LDS char* vl = (const MLA_LDS char*)lds_v[buf];
    // ---- S^T[32 tokens x 32 rows]: lane holds row r32, tokens 8(i/4) + 4hi + i%4
    f32x16 s = {};
#pragma unroll
    for (int st = 0; st < KS; ++st) {
      const bf16x8 a = lds_read_b128(kl, r32 * DK * 2 + 16 * pf_chunk<KCH>(r32, 2 * st + hi));
      s = mfma_32x32x16(a, qf[st], s);
    }
    float mt = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int t = TT * j + 8 * (i >> 2) + 4 * hi + (i & 3);
      const float v = t <= pos ? s[i] * scale_log2 : -INFINITY;
      s[i] = v;
      mt = fmaxf(mt, v);
    }
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const float m_new = fmaxf(m_run, mt);
    // a row with no token so far keeps m = -inf: its weights are 0 and nothing is rescaled
    const float alpha = m_new == -INFINITY ? 1.f : exp2f_fast(m_run - m_new);
    m_run = m_new;
#pragma unroll
    for (int nb = 0; nb < DV / 32; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[nb][i] *= alpha;
    float lsum = 0.f;
    bf16x8 pa[2];  // contraction block kk: tokens 16kk + 8(j/4) + 4hi + j%4
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const float x = s[8 * kk + jj];
        const __bf16 p = (__bf16)(x == -INFINITY ? 0.f : exp2f_fast(x - m_new));
        pa[kk][jj] = p;
        lsum += (float)p;
      }
    l_lane = l_lane * alpha + lsum;
    // ---- O^T[DV x 32 rows] += V^T P^T: the value operand holds, for lane column
    // 32nb + (l & 31), the tokens of contraction block kk in the order above (two transposing
    // reads of four consecutive tokens each)
#pragma unroll
    for (int nb = 0; nb < DV / 32; ++nb)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        bf16x4 v2[2];
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          const int t = 16 * kk + 8 * p + 4 * (G16 >> 1) + (q16 >> 2);
          const int c0 = 32 * nb + 16 * (G16 & 1) + 4 * (q16 & 3);  // first of 4 columns
          v2[p] = lds_read_tr16(vl, t * DV * 2 + 16 * pf_chunk<VCH>(t, c0 >> 3) + (c0 & 7) * 2);
        }
        acc[nb] = mfma_32x32x16(cat4(v2[0], v2[1]), pa[kk], acc[nb]);
      }
    if (j + 1 < ntiles) {
      // the other buffer was last read in the previous tile, before the barrier that ended it
      store_tile(buf ^ 1);
      __syncthreads();
    }
  }
  // ---- normalise and write: lane holds row qi, columns 32nb + 8(i/4) + 4hi + i%4
  const float lt = l_lane + __shfl_xor(l_lane, 32, 64);
  if (qi < T) {
    const float il = lt > 0.f ? 1.f / lt : 0.f;
    uint16_t* o = out + (((size_t)b * T + qi) * H + h) * DV;
#pragma unroll
    for (int nb = 0; nb < DV / 32; ++nb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x16& a = acc[nb];
        const u32x2 w = {pack_bf16x2(a[4 * g] * il, a[4 * g + 1] * il),
                         pack_bf16x2(a[4 * g + 2] * il, a[4 * g + 3] * il)};
        *reinterpret_cast<u32x2*>(o + 32 * nb + 8 * g + 4 * hi) = w;
      }
    if (lse_out && hi == 0)
      lse_out[((size_t)b * T + qi) * H + h] =
          lt > 0.f ? (m_run + log2f_fast(lt)) * kLn2 : -INFINITY;
  }
}

// ---------------------------------------------------------------- attention, DeepSeek widths
// The same computation as prefill_attn_kernel for d_nope = d_v = 128, d_rope = 64, with a
// work group per (sequence, head, 256 query rows): eight waves of 32 rows, so that at T <= 256
// a head's keys and values are read once. The 32-token tiles stream straight into a six-entry
// LDS ring (direct global->LDS loads, five tiles in flight) issued by waves 0..3, five load
// instructions each per tile: an entry is [K_nope 32 x 256 B | k_R 32 x 128 B | V 32 x 256 B],
// each row's 16-byte chunks XOR-swizzled by the row (K_nope and V by r % 16, k_R by (r / 2) %
// 8) so that the MFMA operand reads of 16 consecutive rows hit distinct banks. A tile's 32
// tokens lie in one 64-token page, whose k_R rows come straight from the paged cache.
// Grid: x = 256-row query block, y = head, z = sequence of the group.
namespace pfa {
constexpr int QB = 256, NT = 512, TT = 32, NBUF = 6;
constexpr int KNB = TT * 256, KRB = TT * 128, VB = TT * 256;  // bytes of an entry's parts
constexpr int ENT = KNB + KRB + VB;                           // 20 KiB
constexpr int IPW = 5;  // load instructions per loading wave per tile (20 KiB / 4 waves)
}  // namespace pfa

// Waits until at most `after` tiles of IPW load instructions each are still in flight
// (after <= NBUF - 2).
template <int A>
__device__ __forceinline__ void pfa_wait_tiles(int after) {
  if (after >= A) wait_vmcnt<A * pfa::IPW>();
  else if constexpr (A > 0) pfa_wait_tiles<A - 1>(after);
}

__global__ void __launch_bounds__(pfa::NT)
prefill_attn_ds_kernel(const uint16_t* __restrict__ q_nope, const uint16_t* __restrict__ q_rope,
                       const char* __restrict__ kv, const int32_t* __restrict__ page_table,
                       const int32_t* __restrict__ seq_lens, int b0, int max_pages,
                       int num_pages, int T, const uint16_t* __restrict__ kbuf,
                       const uint16_t* __restrict__ vbuf, int smax, float scale_log2,
                       uint16_t* __restrict__ out, float* __restrict__ lse_out) {
  using namespace pfa;
  constexpr int H = 128, DN = 128, DR = 64, DV = 128, DC = 512;
  constexpr int KS = (DN + DR) / 16;  // 32x32x16 steps over the score contraction (12)
  constexpr int ROWB = (DC + DR) * 2;
  static_assert(ENT % 1024 == 0 && 4 * IPW * 1024 == ENT, "entry of whole KiB, 4 loaders");
  __shared__ __attribute__((aligned(1024))) char lds_ring[NBUF * ENT];
  MLA_LDS char* const ring = (MLA_LDS char*)lds_ring;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int sl = blockIdx.z, b = b0 + sl, h = blockIdx.y;
  const int S = min(clamp_len(ld_uniform(seq_lens + b), max_pages), smax);
  const int i0 = blockIdx.x * QB;  // first query row of the block
  // the block's last row sits at position S - T + min(T - 1, i0 + QB - 1): tokens past it are
  // masked for every row of the block (so ntok <= S)
  const int last = S - T + min(T - 1, i0 + QB - 1);
  const int ntok = last + 1 > 0 ? last + 1 : 0;
  const int ntiles = (ntok + TT - 1) / TT;

  // ---- tile loads (waves 0..3): instruction u of wave w is number w + 4u of the tile's 20:
  // u = 0, 1 -> K_nope rows 4i .. 4i+3 (i = w + 4u), u = 2 -> k_R rows 8w .. 8w+7,
  // u = 3, 4 -> V rows 4i .. 4i+3 (i = w + 4u - 12). Lane l fills LDS slot l of the KiB; it
  // loads the chunk that the row's swizzle puts there. Rows past the sequence's end repeat
  // its last token (masked).
  const bool loader = wave < 4;
  const char* const kb = reinterpret_cast<const char*>(kbuf + ((size_t)sl * H + h) * smax * DN);
  const char* const vb = reinterpret_cast<const char*>(vbuf + ((size_t)sl * H + h) * smax * DV);
  const int32_t* const prow = page_table + (size_t)b * max_pages;
  auto issue_tile = [&](int j) {
    MLA_LDS char* const ent = ring + (j % NBUF) * ENT;
    int page = ld_uniform(prow + min(TT * j / kPage, max_pages - 1));
    page = page < 0 ? 0 : (page >= num_pages ? num_pages - 1 : page);
    const char* const rbase = kv + (size_t)page * kPage * ROWB;
#pragma unroll
    for (int u = 0; u < IPW; ++u) {
      if (u < 2 || u > 2) {  // K_nope (u < 2) or V (u > 2): four 256-byte rows per KiB
        const int i = u < 2 ? wave + 4 * u : wave + 4 * u - 12;
        const int r = 4 * i + (lane >> 4), t = min(TT * j + r, S - 1);
        const int c = (lane & 15) ^ (r & 15);
        if (u < 2) load_lds_16(kb, (uint32_t)(t * 256 + 16 * c), ent + 1024 * i);
        else load_lds_16(vb, (uint32_t)(t * 256 + 16 * c), ent + KNB + KRB + 1024 * i);
      } else {  // k_R: eight 128-byte rows per KiB, from the page's cache rows
        const int r = 8 * wave + (lane >> 3), t = min(TT * j + r, S - 1);
        const int c = (lane & 7) ^ ((r >> 1) & 7);
        load_lds_16(rbase, (uint32_t)((t % kPage) * ROWB + DC * 2 + 16 * c),
                    ent + KNB + 1024 * wave);
      }
    }
  };
  int issued = 0;
  if (loader)
    for (; issued < NBUF - 1 && issued < ntiles; ++issued) issue_tile(issued);

  const int r32 = lane & 31, hi = lane >> 5;
  const int G16 = lane >> 4, q16 = lane & 15;
  const int qi = i0 + 32 * wave + r32;        // this lane's query row
  const int qc = qi < T ? qi : T - 1;         // (rows past T load a valid row, write nothing)
  const int pos = S - T + qi;                 // its position: attends to tokens 0 .. pos
  // query operand: B of S^T = K Q^T, lane = row r32, dims 16s + 8hi .. +8. Waiting for it
  // (the loads complete in order) also lands the tiles issued above.
  bf16x8 qf[KS];
  {
    const uint16_t* qn = q_nope + (((size_t)b * T + qc) * H + h) * DN;
    const uint16_t* qr = q_rope + (((size_t)b * T + qc) * H + h) * DR;
#pragma unroll
    for (int st = 0; st < KS; ++st) {
      const int d = 16 * st + 8 * hi;
      qf[st] = d < DN ? *reinterpret_cast<const bf16x8*>(qn + d)
                      : *reinterpret_cast<const bf16x8*>(qr + (d - DN));
    }
#pragma unroll
    for (int st = 0; st < KS; ++st) settle(qf[st]);
  }
  wait_vmcnt<0>();
  block_sync();  // tile 0 (and those after it) landed

  f32x16 acc[DV / 32] = {};
  float m_run = -INFINITY, l_lane = 0.f;
  for (int j = 0; j < ntiles; ++j) {
    // tile j + NBUF - 1 into the entry of tile j - 1, free since the barrier that ended it
    if (loader && issued < ntiles) issue_tile(issued++);
    const MLA_LDS char* const ent = ring + (j % NBUF) * ENT;
    // ---- S^T[32 tokens x 32 rows]: lane holds row r32, tokens 8(i/4) + 4hi + i%4
    f32x16 s = {};
#pragma unroll
    for (int st = 0; st < KS; ++st) {
      const int c = 2 * st + hi;
      const bf16x8 a = st < DN / 16
          ? lds_read_b128(ent, r32 * 256 + 16 * (c ^ (r32 & 15)))
          : lds_read_b128(ent, KNB + r32 * 128 + 16 * ((c - DN / 8) ^ ((r32 >> 1) & 7)));
      s = mfma_32x32x16(a, qf[st], s);
    }
    float mt = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int t = TT * j + 8 * (i >> 2) + 4 * hi + (i & 3);
      const float v = t <= pos ? s[i] * scale_log2 : -INFINITY;
      s[i] = v;
      mt = fmaxf(mt, v);
    }
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const float m_new = fmaxf(m_run, mt);
    // a row with no token so far keeps m = -inf: its weights are 0 and nothing is rescaled
    const float alpha = m_new == -INFINITY ? 1.f : exp2f_fast(m_run - m_new);
    m_run = m_new;
#pragma unroll
    for (int nb = 0; nb < DV / 32; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[nb][i] *= alpha;
    float lsum = 0.f;
    bf16x8 pa[2];  // contraction block kk: tokens 16kk + 8(j/4) + 4hi + j%4
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const float x = s[8 * kk + jj];
        const __bf16 p = (__bf16)(x == -INFINITY ? 0.f : exp2f_fast(x - m_new));
        pa[kk][jj] = p;
        lsum += (float)p;
      }
    l_lane = l_lane * alpha + lsum;
    // ---- O^T[DV x 32 rows] += V^T P^T (transposing reads of four consecutive tokens)
#pragma unroll
    for (int nb = 0; nb < DV / 32; ++nb)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        bf16x4 v2[2];
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          const int t = 16 * kk + 8 * p + 4 * (G16 >> 1) + (q16 >> 2);
          const int c0 = 32 * nb + 16 * (G16 & 1) + 4 * (q16 & 3);  // first of 4 columns
          v2[p] = lds_read_tr16(ent, KNB + KRB + t * 256 + 16 * ((c0 >> 3) ^ (t & 15)) +
                                         (c0 & 7) * 2);
        }
        acc[nb] = mfma_32x32x16(cat4(v2[0], v2[1]), pa[kk], acc[nb]);
      }
    if (j + 1 < ntiles) {
      // tile j+1 landed: the loading waves wait until only the tiles after it are in flight
      if (loader) pfa_wait_tiles<NBUF - 2>(issued - (j + 2));
      block_sync();
    }
  }
  // ---- normalise and write: lane holds row qi, columns 32nb + 8(i/4) + 4hi + i%4
  const float lt = l_lane + __shfl_xor(l_lane, 32, 64);
  if (qi < T) {
    const float il = lt > 0.f ? 1.f / lt : 0.f;
    uint16_t* o = out + (((size_t)b * T + qi) * H + h) * DV;
#pragma unroll
    for (int nb = 0; nb < DV / 32; ++nb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x16& a = acc[nb];
        const u32x2 w = {pack_bf16x2(a[4 * g] * il, a[4 * g + 1] * il),
                         pack_bf16x2(a[4 * g + 2] * il, a[4 * g + 3] * il)};
        *reinterpret_cast<u32x2*>(o + 32 * nb + 8 * g + 4 * hi) = w;
      }
    if (lse_out && hi == 0)
      lse_out[((size_t)b * T + qi) * H + h] =
          lt > 0.f ? (m_run + log2f_fast(lt)) * kLn2 : -INFINITY;
  }
}

// ---------------------------------------------------------------- launch
hipError_t launch_prefill(int shape, const void* q_nope, const void* q_rope, const void* W_UK,
                          const void* W_UV, const void* kv, const int32_t* page_table,
                          const int32_t* seq_lens, int B, int T, int max_pages, int num_pages,
                          int smax, int group, float scale_log2, void* W_UVt, void* kbuf,
                          void* vbuf, void* out, float* lse_out, const Launch& L) {
  auto run = [&](auto H_, auto DN_, auto DC_, auto DR_, auto DV_) -> hipError_t {
    constexpr int H = decltype(H_)::value, DN = decltype(DN_)::value, DC = decltype(DC_)::value;
    constexpr int DR = decltype(DR_)::value, DV = decltype(DV_)::value;
    hipError_t e = launch_kernel(transpose_wuv_kernel<DC, DV>, dim3(DV / 32, DC / 32, H),
                                 dim3(256), L, (const uint16_t*)W_UV, (uint16_t*)W_UVt);
    if (e != hipSuccess) return e;
    const Launch Ls{L.stream};
    for (int b0 = 0; b0 < B; b0 += group) {
      const int g = min(group, B - b0);
      e = launch_kernel(decompress_kernel<H, DN, DC, DR, DV>,
                        dim3(2 * H, (smax + pf::DTOK - 1) / pf::DTOK, g), dim3(pf::DNT), Ls,
                        (const char*)kv, page_table, seq_lens, b0, max_pages, num_pages,
                        (const uint16_t*)W_UK, (const uint16_t*)W_UVt, (uint16_t*)kbuf,
                        (uint16_t*)vbuf, smax);
      if (e != hipSuccess) return e;
      if constexpr (H == 128 && DN == 128 && DR == 64 && DV == 128)
        e = launch_kernel(prefill_attn_ds_kernel, dim3((T + pfa::QB - 1) / pfa::QB, H, g),
                          dim3(pfa::NT), Ls, (const uint16_t*)q_nope, (const uint16_t*)q_rope,
                          (const char*)kv, page_table, seq_lens, b0, max_pages, num_pages, T,
                          (const uint16_t*)kbuf, (const uint16_t*)vbuf, smax, scale_log2,
                          (uint16_t*)out, lse_out);
      else
        e = launch_kernel(prefill_attn_kernel<H, DN, DC, DR, DV>,
                          dim3((T + pf::QB - 1) / pf::QB, H, g), dim3(pf::NT), Ls,
                          (const uint16_t*)q_nope, (const uint16_t*)q_rope, (const char*)kv,
                          page_table, seq_lens, b0, max_pages, num_pages, T,
                          (const uint16_t*)kbuf, (const uint16_t*)vbuf, smax, scale_log2,
                          (uint16_t*)out, lse_out);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  };
  using std::integral_constant;
  if (shape == kShapeDeepSeek)
    return run(integral_constant<int, 128>{}, integral_constant<int, 128>{},
               integral_constant<int, 512>{}, integral_constant<int, 64>{},
               integral_constant<int, 128>{});
  return run(integral_constant<int, 32>{}, integral_constant<int, 120>{},
             integral_constant<int, 64>{}, integral_constant<int, 8>{},
             integral_constant<int, 128>{});
}

}  // namespace mla
