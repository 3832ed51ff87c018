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
//   decompress: per (sequence, 128 tokens, head, K or V): out^T[128 columns x 128 tokens] =
//     W[h] (columns x d_c) . c_KV^T, 32x32x16 bf16 MFMA over d_c in chunks of 32 staged in LDS
//     (double-buffered through registers), rows of the page-table-addressed cache gathered
//     directly; bf16 out into the workspace ([token][head][width] per sequence).
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
constexpr int TOK = 128;      // decompress: tokens per work group
constexpr int COLS = 128;     // decompress: output columns per work group (one K or V block)
constexpr int KC = 32;        // decompress: contraction chunk
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
// Grid: x = 128-token block of the sequence, y = 2*h + part (part 0: K_nope of head h from
// W_UK[h], rows d < DN; part 1: V of head h from W_UVt[h]), z = sequence of the group.
template <int H, int DN, int DC, int DR, int DV>
__global__ void __launch_bounds__(pf::NT)
decompress_kernel(const char* __restrict__ kv, const int32_t* __restrict__ page_table,
                  const int32_t* __restrict__ seq_lens, int b0, int max_pages, int num_pages,
                  const uint16_t* __restrict__ W_UK, const uint16_t* __restrict__ W_UVt,
                  uint16_t* __restrict__ kbuf, uint16_t* __restrict__ vbuf, int smax) {
  using namespace pf;
  constexpr int ROWB = (DC + DR) * 2;  // bytes per cache token row
  constexpr int NCH = KC * 2 / 16;     // 16-byte chunks per LDS row (4)
  static_assert(DC % KC == 0 && DN <= COLS && DV == COLS, "shape");
  __shared__ __attribute__((aligned(16))) char lds_w[2][COLS * KC * 2];
  __shared__ __attribute__((aligned(16))) char lds_a[2][TOK * KC * 2];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int sl = blockIdx.z, b = b0 + sl;
  const int h = blockIdx.y >> 1, part = blockIdx.y & 1;
  const int t0 = blockIdx.x * TOK;
  // S_b within the page table and within the rows the workspace keeps per sequence (smax,
  // the dims' max_seq_len: S_b <= max_seq_len is the caller's contract, enforced here)
  const int S = min(clamp_len(seq_lens[b], max_pages), smax);
  if (t0 >= S) return;
  const int rows_w = part == 0 ? DN : DV;
  const uint16_t* W = part == 0 ? W_UK + (size_t)h * DN * DC : W_UVt + (size_t)h * DV * DC;

  // this thread's two W pieces and two A pieces per chunk: 512 pieces of 16 bytes each
  const uint16_t* wsrc[2];
  const uint16_t* asrc[2];
  uint32_t wdst[2], adst[2];
  bool wok[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int p = tid + NT * k, r = p >> 2, c = p & 3;
    wok[k] = r < rows_w;
    wsrc[k] = W + (size_t)(wok[k] ? r : 0) * DC + 8 * c;
    wdst[k] = (uint32_t)(r * KC * 2 + 16 * pf_chunk<NCH>(r, c));
    int t = t0 + r;
    t = t < S ? t : S - 1;  // rows past the end repeat the last token (their outputs are unused)
    int page = page_table[(size_t)b * max_pages + t / kPage];
    page = page < 0 ? 0 : (page >= num_pages ? num_pages - 1 : page);
    asrc[k] = reinterpret_cast<const uint16_t*>(kv + ((size_t)page * kPage + t % kPage) * ROWB) +
              8 * c;
    adst[k] = (uint32_t)(r * KC * 2 + 16 * pf_chunk<NCH>(r, c));
  }
  u32x4 wreg[2], areg[2];
  auto load_chunk = [&](int kc) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      wreg[k] = wok[k] ? *reinterpret_cast<const u32x4*>(wsrc[k] + kc * KC) : u32x4{0, 0, 0, 0};
      areg[k] = *reinterpret_cast<const u32x4*>(asrc[k] + kc * KC);
    }
  };
  auto store_chunk = [&](int buf) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      *reinterpret_cast<MLA_LDS u32x4*>((MLA_LDS char*)lds_w[buf] + wdst[k]) = wreg[k];
      *reinterpret_cast<MLA_LDS u32x4*>((MLA_LDS char*)lds_a[buf] + adst[k]) = areg[k];
    }
  };

  // wave: columns 64 (wave & 1) .. +64, tokens 64 (wave >> 1) .. +64, as 2 x 2 blocks of 32
  const int mw = 64 * (wave & 1), nw = 64 * (wave >> 1);
  const int r32 = lane & 31, hi = lane >> 5;
  f32x16 acc[2][2] = {};
  load_chunk(0);
  store_chunk(0);
  __syncthreads();
  constexpr int NCHUNK = DC / KC;
  for (int kc = 0; kc < NCHUNK; ++kc) {
    const int buf = kc & 1;
    if (kc + 1 < NCHUNK) load_chunk(kc + 1);
    const MLA_LDS char* wl = (const MLA_LDS char*)lds_w[buf];
    const MLA_LDS char* al = (const MLA_LDS char*)lds_a[buf];
#pragma unroll
    for (int ks = 0; ks < KC / 16; ++ks) {
      bf16x8 wa[2], ab[2];
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int r = mw + 32 * m + r32;
        wa[m] = lds_read_b128(wl, r * KC * 2 + 16 * pf_chunk<NCH>(r, 2 * ks + hi));
      }
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        const int r = nw + 32 * n + r32;
        ab[n] = lds_read_b128(al, r * KC * 2 + 16 * pf_chunk<NCH>(r, 2 * ks + hi));
      }
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int n = 0; n < 2; ++n) acc[m][n] = mfma_32x32x16(wa[m], ab[n], acc[m][n]);
    }
    if (kc + 1 < NCHUNK) {
      store_chunk(buf ^ 1);  // the other buffer: its last reads were before the last barrier
      __syncthreads();
    }
  }
  // out^T block (m, n): lane holds token nw + 32n + r32 and columns mw + 32m + 8(i/4) + 4hi
  // + i%4; four consecutive columns go out as one 8-byte store
  const int width = part == 0 ? DN : DV;
  uint16_t* dst = part == 0 ? kbuf : vbuf;
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const int t = t0 + nw + 32 * n + r32;
    if (t >= S) continue;
    uint16_t* row = dst + (((size_t)sl * smax + t) * H + h) * width;
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = mw + 32 * m + 8 * g + 4 * hi;
        if (col + 4 > width) continue;
        const f32x16& o = acc[m][n];
        const u32x2 w = {pack_bf16x2(o[4 * g], o[4 * g + 1]), pack_bf16x2(o[4 * g + 2], o[4 * g + 3])};
        *reinterpret_cast<u32x2*>(row + col) = w;
      }
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
        src = vbuf + (((size_t)sl * smax + t) * H + h) * DV + 8 * c;
      } else if (c < NCH_N) {
        src = kbuf + (((size_t)sl * smax + t) * H + h) * DN + 8 * c;
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
                        dim3((smax + pf::TOK - 1) / pf::TOK, 2 * H, g), dim3(pf::NT), Ls,
                        (const char*)kv, page_table, seq_lens, b0, max_pages, num_pages,
                        (const uint16_t*)W_UK, (const uint16_t*)W_UVt, (uint16_t*)kbuf,
                        (uint16_t*)vbuf, smax);
      if (e != hipSuccess) return e;
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
