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
// A work group has 8 waves (two per SIMD) and streams 32-token tiles (36 KiB) through 3 LDS
// buffers (2 in flight). For its 64 heads, per tile:
//   scores  S^T[32 tok x 32 heads] per head block hb (2 per group). The 576-wide contraction is
//           split over four waves kq on 8-chunk boundaries (latent 128kq..128kq+127 plus RoPE
//           16kq..16kq+15): 9 MFMA 32x32x16 each with the wave's query slice (36 VGPRs) held
//           for the segment. Partial scores are summed through LDS: wave kq owns tokens
//           8kq..8kq+7 and receives the other three partials for them.
//   softmax each wave turns its 8 tokens of a head (4 per lane) into bf16 weights P in LDS.
//           The four waves share a per-head reference max fixed on the segment's first tile;
//           only when a tile beats it by more than 2^64 do they agree on a new one and rescale.
//   values  O[64 heads x 64 latent cols of this wave] += P[64 x 32] * tile[32 x 64 cols],
//           8 MFMA 32x32x16, value operand by transposing LDS reads.
// Two work-group barriers per tile: after the scores (partials visible, the oldest buffer free
// for the next prefetch) and after the softmax (P and the next tile visible).
namespace ds {
constexpr int H = 128, HG = 64, DC = 512, DR = 64, DK = DC + DR, ROWB = DK * 2;
constexpr int NBUF = 3;
constexpr int NW = 8;        // waves per work group
constexpr int PPITCH = 80;   // bytes per head row of P (32 bf16 + 16 pad: conflict-free reads)
constexpr int KSTEPS = 9;    // score MFMA steps per wave: a quarter of the 576-wide contraction
using Tile = PagedTile<kSub, ROWB>;
constexpr int IPW = Tile::INSTR / 4;  // load instructions per loading wave (waves 0..3)
constexpr float kRescale = 64.f;      // log2 headroom before the running max must move
}  // namespace ds

template <int N>
__device__ __forceinline__ void wait_tiles_after(int tiles_after) {
  // tile loads complete in order: at most `tiles_after` later tiles (N instructions each) pending
  if (tiles_after >= 1) wait_vmcnt<N>();
  else wait_vmcnt<0>();
}

__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_deepseek_kernel(const uint16_t* __restrict__ q_abs, const uint16_t* __restrict__ q_rope,
                     const char* __restrict__ kv, const int32_t* __restrict__ page_table,
                     const int32_t* __restrict__ seq_lens, int B, int max_pages, int num_pages,
                     const Plan* __restrict__ plan, float scale_log2,
                     uint16_t* __restrict__ part_o, float* __restrict__ part_lse) {
  using namespace ds;
  static_assert(NBUF == 3, "wait_tiles_after covers one later tile");
  __shared__ __attribute__((aligned(1024))) char lds_tiles[NBUF * Tile::BYTES];
  // partial scores: [head block][owner kq][slot (source kq skipping the owner)][lane]
  __shared__ __attribute__((aligned(16))) f32x4 lds_x[2][4][3][64];
  __shared__ __attribute__((aligned(16))) char lds_p[HG * PPITCH];
  __shared__ __attribute__((aligned(16))) float lds_alpha[HG];
  __shared__ __attribute__((aligned(16))) float lds_invl[HG];
  __shared__ __attribute__((aligned(16))) float lds_m[2][4][32];  // [hb][kq][head] maxima
  __shared__ __attribute__((aligned(16))) float lds_l[2][4][32];  // [hb][kq][head] row sums
  __shared__ int lds_flag[NW];

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

  MLA_LDS char* tiles = (MLA_LDS char*)lds_tiles;
  MLA_LDS char* pbuf = (MLA_LDS char*)lds_p;

  const int t32 = lane & 31, hi = lane >> 5;
  const int hb = wave & 1, kq = wave >> 1;
  const int hloc = 32 * hb + t32;   // local head (0..63) whose scores this lane holds
  const int head = HG * hh + hloc;  // global head
  const int G16 = lane >> 4, q16 = lane & 15;
  const bool loader = wave < 4;     // waves 0..3 issue the tile loads, 9 instructions each

  uint32_t dmo[IPW];
#pragma unroll
  for (int k = 0; k < IPW; ++k) dmo[k] = Tile::src_off((wave & 3) + 4 * k, lane, kSub);
  // score operand: row t32, latent chunks 16kq + 2st + hi (st < 8), RoPE chunk 64 + 2kq + hi
  const int fs = Tile::swz(t32);
  uint32_t oq[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) oq[s] = t32 * ROWB + 16 * (16 * kq + ((2 * s + hi) ^ fs));
  const uint32_t orp = t32 * ROWB + 16 * (64 + ((2 * kq + hi) ^ fs));
  // value operand (transposing reads): rows 16*ks + 8*(G16/2) + 4*hf + q16/4, latent columns
  // 64*wave + 32*nb + 16*(G16%2) + 4*(q16%4); the swizzle of those rows does not depend on ks
  uint32_t ov[2][2];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int t = 8 * (G16 >> 1) + 4 * hf + (q16 >> 2);
      const int low = 4 * nb + 2 * (G16 & 1) + ((q16 >> 1) & 1);
      ov[hf][nb] = t * ROWB + 16 * (8 * wave + (low ^ Tile::swz(t))) + 8 * (q16 & 1);
    }
  const uint32_t pw = hloc * PPITCH + 16 * kq + 8 * hi;  // P write: this wave's 4 tokens
  const uint32_t pr = t32 * PPITCH + 16 * hi;            // P read: + 32*PPITCH*mb + 32*ks

  auto issue_tile = [&](const Cursor& c, int buf) {
    if (!loader) return;
    const char* base =
        Tile::tile_base(kv, page_table + (size_t)c.b * max_pages, c.j, num_pages);
    Tile::issue<4>(base, min(kSub, c.S - c.j * kSub), dmo, tiles + buf * Tile::BYTES,
                   wave & 3, lane);
  };

  bf16x8 qf[KSTEPS];
  auto load_queries = [&](int b) {  // this wave's query slice, loads completed here
    const uint16_t* qa = q_abs + ((size_t)b * H + head) * DC + 128 * kq + 8 * hi;
    const uint16_t* qr = q_rope + ((size_t)b * H + head) * DR + 16 * kq + 8 * hi;
#pragma unroll
    for (int st = 0; st < 8; ++st) qf[st] = *reinterpret_cast<const bf16x8*>(qa + 16 * st);
    qf[8] = *reinterpret_cast<const bf16x8*>(qr);
#pragma unroll
    for (int st = 0; st < KSTEPS; ++st) settle(qf[st]);
  };

  Cursor cc;
  {
    const int b0 = find_seq(off, B, total, u0);
    cursor_at(cc, b0, u0 - ld_uniform(off + b0), off, seq_lens, B, total, max_pages);
  }
  load_queries(cc.b);
  Cursor lc = cc;
  int issued = 0;
  for (; issued < NBUF - 1 && issued < n; ++issued) {
    issue_tile(lc, issued);
    cursor_next(lc, off, seq_lens, B, total, max_pages);
  }
  wait_tiles_after<IPW>(issued - 1);
  block_sync();

  f32x16 acc[2][2];
  int it = 0;
  bool first_segment = true;
  while (it < n) {
    const int j0 = cc.j, S = cc.S;
    const int seg = min(cc.nj - cc.j, n - it);
    if (!first_segment) load_queries(cc.b);
    first_segment = false;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = f32x16{};
    float m_ref = -INFINITY, l_lane = 0.f;

    for (int k = 0; k < seg; ++k, ++it) {
      const MLA_LDS char* kb = tiles + (it % NBUF) * Tile::BYTES;
      // ---- partial scores over this wave's quarter of the contraction
      bf16x8 a[KSTEPS];
#pragma unroll
      for (int st = 0; st < 8; ++st) a[st] = lds_read_b128(kb, oq[st & 3] + 128 * (st >> 2));
      a[8] = lds_read_b128(kb, orp);
      f32x16 sc = {};
#pragma unroll
      for (int st = 0; st < KSTEPS; ++st) sc = mfma_32x32x16(a[st], qf[st], sc);
      // hand each other wave of the head block the partials of its 4 rows (rows 4q..4q+3)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (q == kq) continue;
        const int slot = q < kq ? kq - 1 : kq;  // this source's slot at owner q
        lds_x[hb][q][slot][lane] = f32x4{sc[4 * q], sc[4 * q + 1], sc[4 * q + 2], sc[4 * q + 3]};
      }
      block_sync();  // partial scores visible; every wave is done with tile it-1
      if (issued < n) {
        issue_tile(lc, issued % NBUF);
        cursor_next(lc, off, seq_lens, B, total, max_pages);
        ++issued;
      }
      // ---- this wave's rows r = 4kq + e: tokens 8kq + 4hi + e
      float v[4];
      {
        f32x4 t4 = {sc[4 * kq], sc[4 * kq + 1], sc[4 * kq + 2], sc[4 * kq + 3]};
#pragma unroll
        for (int sl = 0; sl < 3; ++sl) t4 += lds_x[hb][kq][sl][lane];
        const int valid = min(kSub, S - (j0 + k) * kSub);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          v[e] = 8 * kq + 4 * hi + e < valid ? t4[e] * scale_log2 : -INFINITY;
      }
      float lm = fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3]));
      lm = fmaxf(lm, __shfl_xor(lm, 32, 64));  // this wave's 8 tokens of the head
      if (k == 0) {  // segment start: the head block agrees on the reference max
        if (hi == 0) lds_m[hb][kq][t32] = lm;
        block_sync();
        m_ref = fmaxf(fmaxf(lds_m[hb][0][t32], lds_m[hb][1][t32]),
                      fmaxf(lds_m[hb][2][t32], lds_m[hb][3][t32]));
      }
      const int need = lm > m_ref + kRescale;  // a running max must move (rare)
      if (lane == 0) lds_flag[wave] = __ballot(need) != 0;
      float lsum = 0.f;
      {
        bf16x4 pv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const __bf16 pb = (__bf16)exp2f_fast(v[e] - m_ref);
          pv[e] = pb;
          lsum += (float)pb;
        }
        *reinterpret_cast<MLA_LDS bf16x4*>(pbuf + pw) = pv;
      }
      if (it + 1 < n) wait_tiles_after<IPW>(issued - it - 2);  // tile it+1 has landed
      block_sync();  // P, flags and tile it+1 visible
      int any = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) any |= lds_flag[w];
      if (any) {
        // rare: agree on new reference maxima, recompute this tile's P, rescale accumulators
        if (hi == 0) lds_m[hb][kq][t32] = lm;
        block_sync();
        const float m_new = fmaxf(fmaxf(m_ref, fmaxf(lds_m[hb][0][t32], lds_m[hb][1][t32])),
                                  fmaxf(lds_m[hb][2][t32], lds_m[hb][3][t32]));
        const float alpha = exp2f_fast(m_ref - m_new);
        m_ref = m_new;
        lsum = 0.f;
        bf16x4 pv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const __bf16 pb = (__bf16)exp2f_fast(v[e] - m_ref);
          pv[e] = pb;
          lsum += (float)pb;
        }
        *reinterpret_cast<MLA_LDS bf16x4*>(pbuf + pw) = pv;
        l_lane *= alpha;
        if (kq == 0 && hi == 0) lds_alpha[hloc] = alpha;
        block_sync();
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const f32x4 a4 = *reinterpret_cast<const MLA_LDS f32x4*>(
                (const MLA_LDS char*)lds_alpha + (32 * mb + 8 * r4 + 4 * hi) * 4);
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
#pragma unroll
              for (int e = 0; e < 4; ++e) acc[mb][nb][4 * r4 + e] *= a4[e];
          }
        if (lane == 0) lds_flag[wave] = 0;
        block_sync();
      }
      l_lane += lsum;

      // ---- values: O[64 heads][this wave's 64 columns] += P * V
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        bf16x8 pa[2], vb[2];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) pa[mb] = lds_read_b128(pbuf, pr + 32 * PPITCH * mb + 32 * ks);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          vb[nb] = cat4(lds_read_tr16(kb, ov[0][nb] + ks * 16 * ROWB),
                        lds_read_tr16(kb, ov[1][nb] + ks * 16 * ROWB));
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
          for (int mb = 0; mb < 2; ++mb) acc[mb][nb] = mfma_32x32x16(pa[mb], vb[nb], acc[mb][nb]);
      }
    }

    // ---- end of segment: normalised partial and its lse
    const int slot = cc.b + g;
    const float lw = l_lane + __shfl_xor(l_lane, 32, 64);  // this wave's 8 tokens per tile
    if (hi == 0) lds_l[hb][kq][t32] = lw;
    block_sync();
    if (kq == 0 && hi == 0) {
      const float lt = lds_l[hb][0][t32] + lds_l[hb][1][t32] + lds_l[hb][2][t32] + lds_l[hb][3][t32];
      lds_invl[hloc] = 1.f / lt;
      part_lse[(size_t)slot * H + head] = (m_ref + log2f_fast(lt)) * kLn2;
    }
    block_sync();
    // Stage the normalised bf16 partial, 32 heads at a time, in the buffer of the segment's
    // last tile (no load targets it before the next tile's barrier), then write it out in
    // 16-byte pieces: rows of 512 latent columns, pitch 1040 bytes.
    {
      constexpr int SPITCH = DC * 2 + 16;
      static_assert(32 * SPITCH <= Tile::BYTES, "staging fits one tile buffer");
      MLA_LDS char* stg = tiles + ((it - 1) % NBUF) * Tile::BYTES;
      uint16_t* po = part_o + ((size_t)slot * H + HG * hh) * DC;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const f32x4 il = *reinterpret_cast<const MLA_LDS f32x4*>(
              (const MLA_LDS char*)lds_invl + (32 * mb + 8 * r4 + 4 * hi) * 4);
#pragma unroll
          for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              *reinterpret_cast<MLA_LDS __bf16*>(
                  stg + (8 * r4 + 4 * hi + e) * SPITCH + (64 * wave + 32 * nb + t32) * 2) =
                  (__bf16)(acc[mb][nb][4 * r4 + e] * il[e]);
        }
        block_sync();
#pragma unroll
        for (int k = 0; k < 4; ++k) {  // 32 rows x 64 pieces of 16 bytes over 512 threads
          const int q = k * 512 + tid, row = q >> 6, piece = q & 63;
          *reinterpret_cast<u32x4*>(po + (size_t)(32 * mb + row) * DC + piece * 8) =
              *reinterpret_cast<const MLA_LDS u32x4*>(stg + row * SPITCH + piece * 16);
        }
        block_sync();
      }
    }
    // next sequence (the loop ends when the unit's range is used up)
    cc.j += seg - 1;
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
constexpr float kRescale = 64.f;  // log2 headroom before the running max must move
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
  uint32_t dmo[IPW];  // lane offsets of a full-tile load
#pragma unroll
  for (int k = 0; k < IPW; ++k) dmo[k] = Tile::src_off(k, lane, TT);
  auto issue = [&](const Cursor& c, int buf) {
    const char* base =
        Tile::tile_base(kv, page_table + (size_t)c.b * max_pages, c.j, num_pages);
    Tile::issue<1>(base, min(TT, c.S - c.j * TT), dmo, tiles + buf * Tile::BYTES, 0, lane);
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
    attn_deepseek_kernel<<<blocks, 64 * ds::NW, 0, stream>>>(
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
