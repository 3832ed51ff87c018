// K2: split-KV MLA attention over the paged latent cache, in latent space.
//
// For every segment (sequence b, a run of its cache tiles owned by one plan unit) and head h:
//   s_t  = scale * (q_abs[b,h] . c_KV[t] + q_rope[b,h] . k_R[t])     (NoPE + RoPE logits,
//          lpnh.cn/news/2494972 S2.1; absorbed NoPE query, bhfrc.com/news/60867 S4 path B)
//   online softmax over the segment's tokens (running max m, running sum l)
//   o[c] = sum_t p_t c_KV[t][c]    (values stay in the 512-d latent space; K/V never expanded,
//          bhfrc.com/news/60867 S1)
// and the segment writes its normalised partial o/l (bf16) and lse = ln sum exp(s) (fp32).
// The combine kernel merges the segments of a sequence and applies W_UV.
//
// Softmax runs in the log2 domain (scale folded with log2 e). The running max is updated
// lazily: a head's reference max only moves when a tile beats it by more than 2^8, so most
// tiles need no rescale of the accumulator; weights stay <= 256, exact in the final ratio.
// p is rounded to bf16 for the value MFMA and l sums the rounded weights, so the weights that
// multiply the values are exactly normalised.
#include "device.h"
#include "kernels.h"
#include "paged_tile.h"

namespace mla {

// ---------------------------------------------------------------- plan cursor
struct Cursor {
  int b;   // sequence
  int j;   // tile index inside the sequence
  int nj;  // tiles of the sequence
  int S;   // clamped sequence length
};

__device__ __forceinline__ int seq_tiles(const int32_t* off, int B, int total, int b) {
  return (b + 1 < B ? ld_uniform(off + b + 1) : total) - ld_uniform(off + b);
}

__device__ __forceinline__ void cursor_at(Cursor& c, int b, int j, const int32_t* off,
                                          const int32_t* seq_lens, int B, int total,
                                          int max_pages) {
  c.b = b;
  c.j = j;
  c.nj = seq_tiles(off, B, total, b);
  c.S = clamp_len(ld_uniform(seq_lens + b), max_pages);
}

__device__ __forceinline__ void cursor_next(Cursor& c, const int32_t* off,
                                            const int32_t* seq_lens, int B, int total,
                                            int max_pages) {
  if (++c.j < c.nj) return;
  int b = c.b + 1;
  while (b < B && seq_tiles(off, B, total, b) == 0) ++b;
  if (b < B) cursor_at(c, b, 0, off, seq_lens, B, total, max_pages);
}

// Sequence holding plan tile u (the unique b with off[b] <= u < off[b+1]).
__device__ __forceinline__ int find_seq(const int32_t* off, int B, int total, int u) {
  int lo = 0, hi = B - 1;  // last b with off[b] <= u
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (ld_uniform(off + mid) <= u) lo = mid; else hi = mid - 1;
  }
  (void)total;
  return lo;
}

// ================================================================ DeepSeek widths
// A tile stream (plan unit) is served by two work groups, one per half of the 128 heads, that
// sit on the same XCD (work groups are dealt to the 8 XCDs round robin, so the pair is
// placed 8 ids apart): the cache crosses HBM once and the second read hits that XCD's L2.
// A work group (4 waves, one per SIMD) streams 32-token tiles (36 KiB) through 4 LDS buffers,
// 3 in flight, and for its 64 heads computes per tile:
//   scores  S^T[32 tok x 32 heads] per head block hb (2 per group); the 576-wide contraction is
//           split between two waves (kh = 0: latent 0..287, kh = 1: latent 288..511 + RoPE),
//           18 MFMA 32x32x16 each, with the wave's query slice (72 VGPRs) held in registers for
//           the whole segment. The kh = 1 wave passes its partial scores through LDS.
//   softmax the kh = 0 wave of a head block finishes the scores (lane = one head x 16 tokens;
//           one exchange with lane^32 completes the tile max) and writes P (bf16) to LDS.
//   values  O[64 heads x 128 latent cols of this wave] += P[64 x 32] * tile[32 x 128 cols],
//           16 MFMA 32x32x16; the tile is read with transposing LDS reads (contraction over
//           tokens). Each wave reads only its quarter of the value columns.
namespace ds {
constexpr int H = 128, HG = 64, DC = 512, DR = 64, DK = DC + DR, ROWB = DK * 2;
constexpr int NBUF = 4;
constexpr int PPITCH = 80;      // bytes per head row of P (32 bf16 + 16 pad: conflict-free reads)
constexpr int KHALF = DK / 2;   // 288: contraction share of one wave
constexpr int KSTEPS = KHALF / 16;
using Tile = PagedTile<kSub, ROWB>;
constexpr int IPW = Tile::INSTR / 4;  // load instructions per wave per tile
constexpr float kRescale = 8.f;
}  // namespace ds

__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
attn_deepseek_kernel(const uint16_t* __restrict__ q_abs, const uint16_t* __restrict__ q_rope,
                     const char* __restrict__ kv, const int32_t* __restrict__ page_table,
                     const int32_t* __restrict__ seq_lens, int B, int max_pages, int num_pages,
                     const Plan* __restrict__ plan, float scale_log2,
                     uint16_t* __restrict__ part_o, float* __restrict__ part_lse) {
  using namespace ds;
  __shared__ __attribute__((aligned(1024))) char lds_tiles[NBUF * Tile::BYTES];
  __shared__ __attribute__((aligned(16))) float lds_x[2][16][64];  // kh=1 partial scores
  __shared__ __attribute__((aligned(16))) char lds_p[HG * PPITCH];
  __shared__ __attribute__((aligned(16))) float lds_alpha[HG];
  __shared__ __attribute__((aligned(16))) float lds_invl[HG];
  __shared__ __attribute__((aligned(16))) int lds_flag[4];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  // work group -> (tile stream g, head half hh); both halves of g share an XCD
  const int x = blockIdx.x;
  const int g = 8 * (x >> 4) + (x & 7), hh = (x >> 3) & 1;
  const int total = ld_uniform(&plan->total), per = ld_uniform(&plan->per);
  const int u0 = g * per;
  const int u1 = min(u0 + per, total);
  if (u0 >= u1) return;
  const int32_t* off = plan_off(plan);
  const int n = u1 - u0;

  Cursor lc;
  {
    const int b0 = find_seq(off, B, total, u0);
    cursor_at(lc, b0, u0 - ld_uniform(off + b0), off, seq_lens, B, total, max_pages);
  }
  Cursor cc = lc;

  MLA_LDS char* tiles = (MLA_LDS char*)lds_tiles;
  MLA_LDS char* pbuf = (MLA_LDS char*)lds_p;

  auto issue = [&](const Cursor& c, int buf) {
    const char* base =
        Tile::tile_base(kv, page_table + (size_t)c.b * max_pages, c.j, num_pages);
    const int valid = min(kSub, c.S - c.j * kSub);
    Tile::issue<4>(base, valid, tiles + buf * Tile::BYTES, wave, lane);
  };

  const int t32 = lane & 31, hi = lane >> 5;
  const int hb = wave & 1, kh = wave >> 1;
  const int hloc = 32 * hb + t32;       // local head (0..63) whose scores this lane holds
  const int head = HG * hh + hloc;      // global head
  const int G16 = lane >> 4, q16 = lane & 15;

  bf16x8 qf[KSTEPS];
  f32x16 acc[2][4];
  float m_used = -INFINITY, l_lane = 0.f;
  // this wave's query slice for sequence b, loads completed here; state reset
  auto start_segment = [&](int b) {
    const uint16_t* qa = q_abs + ((size_t)b * H + head) * DC + 8 * hi;
    const uint16_t* qr = q_rope + ((size_t)b * H + head) * DR + 8 * hi;
#pragma unroll
    for (int st = 0; st < KSTEPS; ++st) {
      const int c = KHALF * kh + 16 * st;  // first latent/RoPE index of the step
      qf[st] = c < DC ? *reinterpret_cast<const bf16x8*>(qa + c)
                      : *reinterpret_cast<const bf16x8*>(qr + (c - DC));
    }
#pragma unroll
    for (int st = 0; st < KSTEPS; ++st) settle(qf[st]);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = f32x16{};
    m_used = -INFINITY;
    l_lane = 0.f;
  };
  start_segment(cc.b);
  bool seg_start = false;

  int issued = 0;
  for (; issued < NBUF - 1 && issued < n; ++issued) {
    issue(lc, issued % NBUF);
    cursor_next(lc, off, seq_lens, B, total, max_pages);
  }

  for (int it = 0; it < n; ++it) {
    if (seg_start) {
      start_segment(cc.b);
      seg_start = false;
    }
    // tile `it` has landed once at most the later tiles' loads are outstanding
    const int after = issued - it - 1;
    if (after >= 2) wait_vmcnt<2 * IPW>();
    else if (after == 1) wait_vmcnt<IPW>();
    else wait_vmcnt<0>();
    block_sync();
    if (issued < n) {
      issue(lc, issued % NBUF);
      cursor_next(lc, off, seq_lens, B, total, max_pages);
      ++issued;
    }
    const MLA_LDS char* kb = tiles + (it % NBUF) * Tile::BYTES;

    // ---- partial scores over this wave's half of the contraction
    f32x16 s = {};
#pragma unroll
    for (int st = 0; st < KSTEPS; ++st)
      s = mfma_32x32x16(lds_read_b128(kb, Tile::lds_off(t32, 2 * (KSTEPS * kh + st) + hi)),
                        qf[st], s);
    if (kh == 1) {
#pragma unroll
      for (int r = 0; r < 16; ++r) lds_x[hb][r][lane] = s[r];
    }
    block_sync();

    // ---- online softmax (log2 domain) by the kh = 0 waves; lane = one head x 16 tokens
    int need = 0;
    float alpha = 1.f;
    if (kh == 0) {
      const int valid = min(kSub, cc.S - cc.j * kSub);
      float mt = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int t = 8 * (r >> 2) + 4 * hi + (r & 3);
        const float v = t < valid ? (s[r] + lds_x[hb][r][lane]) * scale_log2 : -INFINITY;
        s[r] = v;
        mt = fmaxf(mt, v);
      }
      mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
      if (m_used == -INFINITY) {
        m_used = mt;
      } else if (mt > m_used + kRescale) {
        alpha = exp2f_fast(m_used - mt);
        m_used = mt;
        need = 1;
      }
      float lsum = 0.f;
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        bf16x4 pv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const __bf16 pb = (__bf16)exp2f_fast(s[4 * r4 + e] - m_used);
          pv[e] = pb;
          lsum += (float)pb;
        }
        *reinterpret_cast<MLA_LDS bf16x4*>(pbuf + hloc * PPITCH + (8 * r4 + 4 * hi) * 2) = pv;
      }
      l_lane = l_lane * alpha + lsum;
      if (hi == 0) lds_alpha[hloc] = alpha;
    }
    if (lane == 0) lds_flag[wave] = __ballot(need) != 0;
    block_sync();
    const int any = lds_flag[0] | lds_flag[1] | lds_flag[2] | lds_flag[3];

    // ---- values: O[64 heads][this wave's 128 columns] += P * V
    if (any) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const f32x4 a4 = *reinterpret_cast<const MLA_LDS f32x4*>(
              (const MLA_LDS char*)lds_alpha + (32 * mb + 8 * r4 + 4 * hi) * 4);
#pragma unroll
          for (int nb = 0; nb < 4; ++nb)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[mb][nb][4 * r4 + e] *= a4[e];
        }
    }
#pragma unroll
    for (int ks = 0; ks < kSub / 16; ++ks) {
      bf16x8 pa[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
        pa[mb] = lds_read_b128(pbuf, (32 * mb + t32) * PPITCH + (16 * ks + 8 * hi) * 2);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        bf16x4 v2[2];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int t = 16 * ks + 8 * (G16 >> 1) + 4 * hf + (q16 >> 2);
          const int c0 = 128 * wave + 32 * nb + 16 * (G16 & 1) + 4 * (q16 & 3);
          v2[hf] = lds_read_tr16(kb, Tile::lds_off(t, c0 >> 3) + (c0 & 7) * 2);
        }
        const bf16x8 vb = cat4(v2[0], v2[1]);
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) acc[mb][nb] = mfma_32x32x16(pa[mb], vb, acc[mb][nb]);
      }
    }

    // ---- end of segment: normalised partial and its lse
    if (it == n - 1 || cc.j == cc.nj - 1) {
      const int slot = cc.b + g;
      if (kh == 0) {
        const float lt = l_lane + __shfl_xor(l_lane, 32, 64);
        if (hi == 0) {
          lds_invl[hloc] = 1.f / lt;
          part_lse[(size_t)slot * H + head] = (m_used + log2f_fast(lt)) * kLn2;
        }
      }
      block_sync();
      uint16_t* po = part_o + ((size_t)slot * H + HG * hh) * DC;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const f32x4 il = *reinterpret_cast<const MLA_LDS f32x4*>(
              (const MLA_LDS char*)lds_invl + (32 * mb + 8 * r4 + 4 * hi) * 4);
#pragma unroll
          for (int nb = 0; nb < 4; ++nb)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int h = 32 * mb + 8 * r4 + 4 * hi + e;
              const int c = 128 * wave + 32 * nb + t32;
              po[(size_t)h * DC + c] = bf16_bits((__bf16)(acc[mb][nb][4 * r4 + e] * il[e]));
            }
        }
      seg_start = true;
    }
    cursor_next(cc, off, seq_lens, B, total, max_pages);
  }
}

// ================================================================ MHA2MLA widths
// H = 32, d_latent = 64, d_rope = 8: a token row is 72 bf16 (144 B), a page 9 KiB. One wave
// holds all 32 heads (queries: 18 VGPRs, accumulator 32), so each wave is its own plan unit
// with a private LDS ring of 4 page buffers (3 pages in flight) and no work-group barriers.
// Per page: scores S^T[64 tok x 32 heads] (2 x (4 MFMA 32x32x16 over the latent + 1 MFMA
// 32x32x8 over RoPE)); the bf16 weights feed the value MFMA straight from registers, by
// numbering the contraction index in the order the score layout holds tokens; values
// O[32 heads x 64 latent] += P * V with 8 MFMA 32x32x16 and transposing reads of V.
namespace m2 {
constexpr int H = 32, DC = 64, DR = 8, DK = DC + DR, ROWB = DK * 2;
constexpr int NBUF = 4;
constexpr int TT = kPage;  // tokens per tile: one page
using Tile = PagedTile<TT, ROWB>;
constexpr int IPW = Tile::INSTR;  // the wave issues the whole tile
constexpr float kRescale = 8.f;
}  // namespace m2

__global__ void __launch_bounds__(256)
attn_mha2mla_kernel(const uint16_t* __restrict__ q_abs, const uint16_t* __restrict__ q_rope,
                    const char* __restrict__ kv, const int32_t* __restrict__ page_table,
                    const int32_t* __restrict__ seq_lens, int B, int max_pages, int num_pages,
                    const Plan* __restrict__ plan, float scale_log2,
                    uint16_t* __restrict__ part_o, float* __restrict__ part_lse) {
  using namespace m2;
  __shared__ __attribute__((aligned(1024))) char lds_tiles[kAttnWavesMha2Mla][NBUF * Tile::BYTES];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform per wave
  const int g = blockIdx.x * kAttnWavesMha2Mla + wave;  // plan unit = wave
  const int total = ld_uniform(&plan->total), per = ld_uniform(&plan->per);
  const int u0 = g * per;
  const int u1 = min(u0 + per, total);
  if (u0 >= u1) return;
  const int32_t* off = plan_off(plan);
  const int n = u1 - u0;
  MLA_LDS char* tiles = (MLA_LDS char*)lds_tiles[wave];

  Cursor lc;
  {
    const int b0 = find_seq(off, B, total, u0);
    cursor_at(lc, b0, u0 - ld_uniform(off + b0), off, seq_lens, B, total, max_pages);
  }
  Cursor cc = lc;
  auto issue = [&](const Cursor& c, int buf) {
    const char* base =
        Tile::tile_base(kv, page_table + (size_t)c.b * max_pages, c.j, num_pages);
    const int valid = min(TT, c.S - c.j * TT);
    Tile::issue<1>(base, valid, tiles + buf * Tile::BYTES, 0, lane);
  };

  const int t32 = lane & 31, hi = lane >> 5;
  const int G16 = lane >> 4, q16 = lane & 15;
  bf16x8 qf[DC / 16];
  i16x4 qr4;
  f32x16 acc[2];
  float m_used = -INFINITY, l_lane = 0.f;
  auto start_segment = [&](int b) {
    const uint16_t* qa = q_abs + ((size_t)b * H + t32) * DC + 8 * hi;
#pragma unroll
    for (int s = 0; s < DC / 16; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(qa + 16 * s);
    qr4 = *reinterpret_cast<const i16x4*>(q_rope + ((size_t)b * H + t32) * DR + 4 * hi);
#pragma unroll
    for (int s = 0; s < DC / 16; ++s) settle(qf[s]);
    settle(qr4);
    acc[0] = f32x16{};
    acc[1] = f32x16{};
    m_used = -INFINITY;
    l_lane = 0.f;
  };
  start_segment(cc.b);
  bool seg_start = false;

  int issued = 0;
  for (; issued < NBUF - 1 && issued < n; ++issued) {
    issue(lc, issued % NBUF);
    cursor_next(lc, off, seq_lens, B, total, max_pages);
  }
  for (int it = 0; it < n; ++it) {
    if (seg_start) {
      start_segment(cc.b);
      seg_start = false;
    }
    const int after = issued - it - 1;
    if (after >= 2) wait_vmcnt<2 * IPW>();
    else if (after == 1) wait_vmcnt<IPW>();
    else wait_vmcnt<0>();
    if (issued < n) {
      issue(lc, issued % NBUF);
      cursor_next(lc, off, seq_lens, B, total, max_pages);
      ++issued;
    }
    const MLA_LDS char* kb = tiles + (it % NBUF) * Tile::BYTES;

    // ---- scores for tokens [32*mb2, 32*mb2 + 32)
    f32x16 s[2];
#pragma unroll
    for (int mb2 = 0; mb2 < 2; ++mb2) {
      const int row = 32 * mb2 + t32;
      f32x16 a = {};
#pragma unroll
      for (int st = 0; st < DC / 16; ++st)
        a = mfma_32x32x16(lds_read_b128(kb, Tile::lds_off(row, 2 * st + hi)), qf[st], a);
      const i16x4 kr = *reinterpret_cast<const MLA_LDS i16x4*>(
          kb + Tile::lds_off(row, DC / 8) + 8 * hi);
      s[mb2] = mfma_32x32x8(kr, qr4, a);
    }
    // ---- online softmax, lane = head t32 x 32 tokens
    const int valid = min(TT, cc.S - cc.j * TT);
    float mt = -INFINITY;
#pragma unroll
    for (int mb2 = 0; mb2 < 2; ++mb2)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int t = 32 * mb2 + 8 * (r >> 2) + 4 * hi + (r & 3);
        const float v = t < valid ? s[mb2][r] * scale_log2 : -INFINITY;
        s[mb2][r] = v;
        mt = fmaxf(mt, v);
      }
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    float alpha = 1.f;
    int need = 0;
    if (m_used == -INFINITY) {
      m_used = mt;
    } else if (mt > m_used + kRescale) {
      alpha = exp2f_fast(m_used - mt);
      m_used = mt;
      need = 1;
    }
    if (__ballot(need)) {  // rescale: O row h (= rows of this lane) by the alpha of head h
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int h = 8 * (r >> 2) + 4 * hi + (r & 3);
        const float a = __shfl(alpha, h, 64);
        acc[0][r] *= a;
        acc[1][r] *= a;
      }
    }
    float lsum = 0.f;
    bf16x8 pa[4];  // value-MFMA operand for contraction block kk = 2*mb2 + half
#pragma unroll
    for (int mb2 = 0; mb2 < 2; ++mb2)
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const __bf16 pb = (__bf16)exp2f_fast(s[mb2][8 * half + j] - m_used);
          pa[2 * mb2 + half][j] = pb;
          lsum += (float)pb;
        }
    l_lane = l_lane * alpha + lsum;
    // ---- values: block kk holds, for lane half hi, the tokens
    //      32*mb2 + 16*half + 8*(j/4) + 4*hi + j%4  (j < 8), the order of the score layout
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int mb2 = kk >> 1, half = kk & 1;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        bf16x4 v2[2];
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          const int t = 32 * mb2 + 16 * half + 8 * p + 4 * (G16 >> 1) + (q16 >> 2);
          const int c0 = 32 * nb + 16 * (G16 & 1) + 4 * (q16 & 3);
          v2[p] = lds_read_tr16(kb, Tile::lds_off(t, c0 >> 3) + (c0 & 7) * 2);
        }
        acc[nb] = mfma_32x32x16(pa[kk], cat4(v2[0], v2[1]), acc[nb]);
      }
    }

    if (it == n - 1 || cc.j == cc.nj - 1) {
      const float lt = l_lane + __shfl_xor(l_lane, 32, 64);
      const int slot = cc.b + g;
      if (hi == 0) part_lse[(size_t)slot * H + t32] = (m_used + log2f_fast(lt)) * kLn2;
      const float il = 1.f / lt;
      uint16_t* po = part_o + (size_t)slot * H * DC;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int h = 8 * (r >> 2) + 4 * hi + (r & 3);
        const float ih = __shfl(il, h, 64);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          po[(size_t)h * DC + 32 * nb + t32] = bf16_bits((__bf16)(acc[nb][r] * ih));
      }
      seg_start = true;
    }
    cursor_next(cc, off, seq_lens, B, total, max_pages);
  }
}

hipError_t launch_attention(int shape, const void* q_abs, const void* q_rope, const void* kv,
                            const int32_t* page_table, const int32_t* seq_lens, int B,
                            int max_pages, int num_pages, const void* plan, int G,
                            float scale_log2, void* part_o, float* part_lse,
                            hipStream_t stream) {
  if (shape == kShapeDeepSeek) {
    // two head halves per tile stream, paired 8 ids apart; ids padded to whole groups of 16
    const int blocks = 16 * ((G + 7) / 8);
    attn_deepseek_kernel<<<blocks, 256, 0, stream>>>(
        (const uint16_t*)q_abs, (const uint16_t*)q_rope, (const char*)kv, page_table, seq_lens,
        B, max_pages, num_pages, (const Plan*)plan, scale_log2, (uint16_t*)part_o, part_lse);
  } else {
    const int blocks = (G + kAttnWavesMha2Mla - 1) / kAttnWavesMha2Mla;
    attn_mha2mla_kernel<<<blocks, 64 * kAttnWavesMha2Mla, 0, stream>>>(
        (const uint16_t*)q_abs, (const uint16_t*)q_rope, (const char*)kv, page_table, seq_lens,
        B, max_pages, num_pages, (const Plan*)plan, scale_log2, (uint16_t*)part_o, part_lse);
  }
  return hipGetLastError();
}

}  // namespace mla
