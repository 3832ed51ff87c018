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
// lazily: a head's reference max only moves when a tile beats it by more than 64 (log2 units),
// so most tiles need no rescale of the accumulator; weights stay below 2^64, far inside the
// fp32 and bf16 range, and the final ratio does not depend on the reference.
// p is rounded to bf16 for the value MFMA. At the DeepSeek widths l sums the rounded weights,
// so the weights that multiply the values are exactly normalised; at the MHA2MLA widths l sums
// the fp32 weights (one instruction less per weight; the two sums differ by bf16 rounding noise
// that averages out over the tokens).
#include <type_traits>

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

__device__ __forceinline__ int seq_tiles(const Plan* plan, int B, int b) {
  const int32_t* off = plan_off(plan);
  return (b + 1 < B ? ld_uniform(off + b + 1) : ld_uniform(&plan->total)) - ld_uniform(off + b);
}

__device__ __forceinline__ void cursor_at(Cursor& c, int b, int j, const Plan* plan,
                                          const int32_t* seq_lens, int B, int max_pages,
                                          int q_len) {
  c.b = b;
  c.j = j;
  c.nj = seq_tiles(plan, B, b);
  c.S = virt_len(clamp_len(ld_uniform(seq_lens + virt_row(b, q_len)), max_pages), b, q_len);
}

// The next tile of the stream (sequences are virtual ones when q_len > 1); the plan is read
// only when a sequence ends.
__device__ __forceinline__ void cursor_next(Cursor& c, const Plan* plan, const int32_t* seq_lens,
                                            int B, int max_pages, int q_len) {
  if (++c.j < c.nj) return;
  int b = c.b + 1;
  while (b < B && seq_tiles(plan, B, b) == 0) ++b;
  if (b < B) cursor_at(c, b, 0, plan, seq_lens, B, max_pages, q_len);
}

// ================================================================ DeepSeek widths
// A tile stream (plan unit) is served by two work groups, one per half of the 128 heads, that
// sit on the same XCD (work groups are dealt to the 8 XCDs round robin, so the pair is placed
// 8 ids apart): the cache crosses HBM once and the second read hits that XCD's L2.
//
// Inside a work group the eight waves form two teams that run one 32-token tile apart, with a
// single work-group barrier per tile:
//   scores  (waves 0..3) wave a holds the whole 576-wide query of 16 heads (72 VGPRs) and
//           computes S^T[32 tok x 16 heads] with 2 x 18 MFMA 16x16x32; the online softmax of
//           those heads is then entirely its own (row maxima by two lane exchanges), and it
//           writes the bf16 weights P, the per-head rescale factors and, at the end of a
//           segment, 1/l and the lse.
//   values  (waves 4..7) wave v accumulates O^T[128 latent columns x 64 heads] += V^T * P^T
//           with 16 MFMA 32x32x16 per tile (value operand by transposing LDS reads), and issues
//           the tile loads; at the end of a segment it normalises, stages its block in the part
//           of the finished tile that only it read, and writes whole rows.
// In round r the score team works on tile r+1 while the value team works on tile r. The ring
// has four 36 KiB buffers: tiles r and r+1 in use, r+2 and r+3 in flight, so a load has two
// rounds to land. P, the rescale factors and 1/l are double buffered by tile parity.
// The reference max of a head is fixed on the segment's first tile and only moves when a tile
// beats it by more than 64 in log2 units (a factor 2^64); the value team then rescales.
//
// FP8 cache (bhfrc.com/news/60867 S1 quantised latent cache, read as FP8 e4m3 with a
// power-of-two scale per token): a token row is [c_KV as FP8 (512 bytes) | k_R bf16 (128
// bytes)], 640 bytes, and a ring entry is a tile's 20 KiB of rows plus its 32 scales. Seven
// entries fit where four bf16 tiles did: tiles r and r+1 in use, r+2 .. r+6 in flight. The MFMA
// operands are formed from the FP8 bytes in registers: a score wave converts its operand (8
// latent values of one token) with that token's scale; a value wave converts its operand (8
// tokens of one latent column, from 8-bit transposing reads) unscaled, and the score wave
// multiplies each token's bf16 weight by the token's scale instead. A power of two moves
// exactly between the two factors, so the products are those over the bf16 cache that holds
// c_KV * scale. At a segment's end a value wave stages its partial in its own 128 columns of
// the finished tile, 64 output columns at a time.
namespace ds {
constexpr int H = 128, HG = 64, DC = 512, DR = 64, DK = DC + DR, ROWB = DK * 2;
constexpr int NW = 8;        // waves per work group: 4 score waves, 4 value waves
constexpr int PPITCH = 80;   // bytes per head row of P (32 bf16 + 16 pad: conflict-free reads)
constexpr int KST = DK / 32; // score MFMA steps (16x16x32) per token block
using Tile = PagedTile<kSub, ROWB>;
constexpr float kRescale = 64.f;      // log2 headroom before the running max must move
constexpr int ROWB8 = DC + 2 * DR;    // FP8 cache: bytes per token row
using Tile8 = PagedTile<kSub, ROWB8>;
constexpr int SCB = 256;              // FP8 cache: bytes of a ring entry's scale block
// Per cache format: ring depth, bytes per ring entry, and load instructions per value wave per
// tile (the FP8 tile's 20 instructions over four waves, plus each wave's load of the scales).
template <bool FP8> struct Ring {
  static constexpr int NBUF = 4, BYTES = Tile::BYTES, TILE_IPW = Tile::INSTR / 4;
  static constexpr int IPW = TILE_IPW;
};
template <> struct Ring<true> {
  static constexpr int NBUF = 7, BYTES = Tile8::BYTES + SCB, TILE_IPW = Tile8::INSTR / 4;
  static constexpr int IPW = TILE_IPW + 1;
};
static_assert(Ring<false>::IPW == 9 && Ring<true>::IPW == 6, "load instructions per wave");
static_assert(Ring<true>::BYTES % 256 == 0, "ring entries start on the same LDS bank");
}  // namespace ds

// Waits until at most `after` tiles of N load instructions each are still in flight, with S
// younger stores also outstanding (a segment's partial, written after the round's tile loads:
// vmcnt counts loads and stores alike, in issue order, so the stores are part of the budget;
// left out, the wait would also hold until the partial is written and drain tile loads that
// may stay in flight). `after` is clamped to MAXA, the most a caller can have in flight (the
// ring depth minus the tiles in use), which also keeps the chain of tests short.
template <int N, int MAXA, int S = 0>
__device__ __forceinline__ void wait_tiles(int after) {
  static_assert(MAXA * N + S < 64, "vmcnt range");
  if (after >= MAXA) wait_vmcnt<MAXA * N + S>();
  else if constexpr (MAXA > 1) wait_tiles<N, MAXA - 1, S>(after);
  else wait_vmcnt<S>();
}

// The absorbed query of one head as hi + lo, two FP8 (e4m3) parts for the block-scaled MFMA.
// raw holds this lane's 128 bf16 elements (chunk j, piece p: elements 128j + 32g4 + 8p .. +8);
// the head's other elements sit in lanes hl + 16, hl + 32 and hl + 48. The hi scale 2^X puts
// the head's largest |q| in [128, 256) (X = floor(log2 max) - 7); hi = RNE(q / 2^X), and lo =
// RNE((q / 2^X - hi) * 16) at scale 2^(X - 4). A bf16 q has 8 significant bits and each part
// keeps 4, so hi + lo is q exactly unless q / 2^X lies below the e4m3 normal range (q below
// about 2^-13 of the head's largest). Codes: qsc[0] for hi, qsc[1] for lo.
__device__ __forceinline__ void split_query_fp8(const u32x4 (&raw)[4][4], i32x8 (&qh)[4],
                                                i32x8 (&ql)[4], int (&qsc)[2]) {
  float am = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t w = raw[j][p][e];
        am = fmaxf(am, fmaxf(fabsf(__builtin_bit_cast(float, w << 16)),
                             fabsf(__builtin_bit_cast(float, w & 0xffff0000u))));
      }
  am = rows4_max(am);
  int ex = 0;
  (void)frexpf(am, &ex);  // am = f 2^ex, f in [0.5, 1): floor(log2 am) = ex - 1
  const int chi = am > 0.f ? min(max(ex + 119, 0), 247) : 127;  // X + 127, X = ex - 8
  const int clo = max(chi - 4, 0);
  const float inv = __builtin_bit_cast(float, (uint32_t)(254 - chi) << 23);        // 2^-X
  const float lmul = __builtin_bit_cast(float, (uint32_t)(127 + chi - clo) << 23);  // 2^(chi-clo)
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    int hw[8] = {0, 0, 0, 0, 0, 0, 0, 0}, lw[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    // elements 8p + 2e and 8p + 2e + 1 (raw word e of piece p) become bytes 2(e & 1) and
    // 2(e & 1) + 1 of word 2p + e/2
    auto split2 = [&](uint32_t w, int& h, int& l, auto sel) {
      const float x0 = __builtin_bit_cast(float, w << 16) * inv;
      const float x1 = __builtin_bit_cast(float, w & 0xffff0000u) * inv;
      h = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, h, decltype(sel)::value);
      const f32x2 hv = __builtin_amdgcn_cvt_pk_f32_fp8(h, decltype(sel)::value);
      l = __builtin_amdgcn_cvt_pk_fp8_f32((x0 - hv[0]) * lmul, (x1 - hv[1]) * lmul, l,
                                          decltype(sel)::value);
    };
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
      for (int e2 = 0; e2 < 2; ++e2) {
        const int k = 2 * p + e2;
        split2(raw[j][p][2 * e2], hw[k], lw[k], std::false_type());
        split2(raw[j][p][2 * e2 + 1], hw[k], lw[k], std::true_type());
      }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      qh[j][k] = hw[k];
      ql[j][k] = lw[k];
    }
  }
  qsc[0] = chi;
  qsc[1] = clo;
}

// FP8 e4m3 -> bf16, 8 values from two words (bytes 0..7 in order), times 2^(exponent of sc)
__device__ __forceinline__ bf16x8 cvt_fp8x8(uint32_t w0, uint32_t w1, float sc) {
  const bf16x2 a0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, sc, false);
  const bf16x2 a1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, sc, true);
  const bf16x2 a2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, sc, false);
  const bf16x2 a3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, sc, true);
  return cat4(__builtin_shufflevector(a0, a1, 0, 1, 2, 3),
              __builtin_shufflevector(a2, a3, 0, 1, 2, 3));
}

template <bool FP8>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_deepseek_kernel(const uint16_t* __restrict__ q_abs, const uint16_t* __restrict__ q_rope,
                     const char* __restrict__ kv, const int32_t* __restrict__ page_table,
                     const int32_t* __restrict__ seq_lens, int B, int max_pages, int q_len,
                     int num_pages,
                     const Plan* __restrict__ plan, int G, float scale_log2,
                     uint16_t* __restrict__ part_o, float* __restrict__ part_lse,
                     const float* __restrict__ kv_scales) {
  using namespace ds;
  using TileL = typename std::conditional<FP8, Tile8, Tile>::type;  // the format as loaded
  constexpr int NBUF = Ring<FP8>::NBUF, LB = Ring<FP8>::BYTES, IPW = Ring<FP8>::IPW;
  constexpr int TIPW = Ring<FP8>::TILE_IPW;  // tile loads per value wave (without the scales)
  __shared__ __attribute__((aligned(1024))) char lds_tiles[NBUF * LB];
  __shared__ __attribute__((aligned(16))) char lds_p[2][HG * PPITCH];
  __shared__ __attribute__((aligned(16))) float lds_alpha[2][HG];  // rescale factor per head
  __shared__ __attribute__((aligned(16))) float lds_invl[2][HG];   // 1/l at a segment's end
  __shared__ __attribute__((aligned(16))) int lds_flag[2][4];      // score wave moved a max

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform per wave
  // work group -> (tile stream g, head half hh); both halves of g share an XCD
  const int x = blockIdx.x;
  // consecutive units (usually the parts of one sequence, which read the same queries) go to
  // the same XCD: ids x with x % 8 == k serve units k*ceil(G/8) ..
  const int per_xcd = (G + 7) >> 3;
  const int g = (x & 7) * per_xcd + (x >> 4), hh = (x >> 3) & 1;
  // the unit record is the only load before the queries and the first tile (ids past G, from
  // padding the grid to whole groups of 16, read the last record and leave)
  const UnitStart us = load_unit(plan, B, g < G ? g : G - 1);
  const int n = g < G ? us.n : 0;  // tiles of this unit
  if (n <= 0) return;
  MLA_LDS char* tiles = (MLA_LDS char*)lds_tiles;
  const Cursor c0 = {us.b, us.j, us.nj, us.S};  // the unit's first tile

  if (wave < 4) {
    // ================= score team: wave a owns local heads 16a .. 16a+15
    const int a = wave;
    const int hl = lane & 15, g4 = lane >> 4;
    const int head = HG * hh + 16 * a + hl;
    // score operand (16x16x32, A = tile rows): token row 16tb + hl, chunk 4s + g4 of step s;
    // with the row swizzle, step s sits at ko[tb][s & 1] + 128 * (s >> 1) (RoPE steps included)
    uint32_t ko[2][2];
    // FP8: the operand of the block-scaled 16x16x128 MFMA over latent chunk j (A = tile rows:
    // token row 16tb + hl, bytes 128j + 32g4 .. +32 of its latent) is the two 16-byte pieces
    // at ka8[tb][0..1] + 128j; RoPE step 16 + q reads the 16 bytes at kr8[tb][q]
    uint32_t ka8[2][2], kr8[2][2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const int r = 16 * tb + hl;
      if constexpr (FP8) {
        const int sw = Tile8::swz(r);
#pragma unroll
        for (int p = 0; p < 2; ++p) ka8[tb][p] = r * ROWB8 + 16 * ((2 * g4 + p) ^ sw);
#pragma unroll
        for (int q = 0; q < 2; ++q) kr8[tb][q] = r * ROWB8 + DC + 16 * ((4 * q + g4) ^ sw);
      } else {
        const int sw = Tile::swz(r);
        ko[tb][0] = r * ROWB + 16 * (g4 ^ sw);
        ko[tb][1] = r * ROWB + 16 * ((4 + g4) ^ sw);
      }
    }
    bf16x8 qf[KST];
    // FP8: the absorbed query of head hl as qh + ql, two FP8 (e4m3) parts with one E8M0 scale
    // each (codes qsc[0], qsc[1]), in the B-operand layout of the block-scaled MFMA (lane: head
    // hl, bytes 32g4 .. +32 of each 128-wide chunk j); the RoPE steps stay bf16 in qf[16..17]
    i32x8 qh[4], ql[4];
    int qsc[2];
    auto load_queries = [&](int b) {  // this wave's 16 queries, loads completed here
      if constexpr (FP8) {
        const uint16_t* qa = q_abs + ((size_t)b * H + head) * DC + 32 * g4;
        const uint16_t* qr = q_rope + ((size_t)b * H + head) * DR + 8 * g4;
        u32x4 raw[4][4];  // chunk j, piece p: elements 128j + 32g4 + 8p .. +8
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int p = 0; p < 4; ++p)
            raw[j][p] = *reinterpret_cast<const u32x4*>(qa + 128 * j + 8 * p);
#pragma unroll
        for (int s = 0; s < 2; ++s) qf[16 + s] = *reinterpret_cast<const bf16x8*>(qr + 32 * s);
        split_query_fp8(raw, qh, ql, qsc);
#pragma unroll
        for (int s = 16; s < KST; ++s) settle(qf[s]);
      } else {
        const uint16_t* qa = q_abs + ((size_t)b * H + head) * DC + 8 * g4;
        const uint16_t* qr = q_rope + ((size_t)b * H + head) * DR + 8 * g4;
#pragma unroll
        for (int s = 0; s < 16; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(qa + 32 * s);
#pragma unroll
        for (int s = 0; s < 2; ++s) qf[16 + s] = *reinterpret_cast<const bf16x8*>(qr + 32 * s);
#pragma unroll
        for (int s = 0; s < KST; ++s) settle(qf[s]);
      }
    };
    load_queries(c0.b);
    block_sync_tagged<0>();  // tile 0 landed

    Cursor ca = c0;
    float m_ref = -INFINITY, l_lane = 0.f;
    for (int r = -1; r < n; ++r) {
      const int t = r + 1;  // this round's tile
      if (t < n) {
        const bool seg_first = t == 0 || ca.j == 0;
        const bool seg_last = t == n - 1 || ca.j == ca.nj - 1;
        if (seg_first && t > 0) load_queries(ca.b);
        const MLA_LDS char* kb = tiles + (t % NBUF) * LB;
        // Token block 0 first, then block 1; each block accumulates in two chains (even and odd
        // steps). Operand reads run one half-block (9 steps) ahead of the MFMAs, and on tiles
        // whose reference max is already set the weights of block 0 are formed while block 1's
        // MFMAs run (scheduling fences and groups keep that order).
        // bf16: the operands as read, nine steps of 16x16x32 per half-block. FP8: half h of a
        // block is latent chunks 2h and 2h+1 (32 bytes a lane each), which feed the
        // block-scaled 16x16x128 MFMA as stored, once against qh and once against ql, and
        // RoPE step h (bf16).
        struct Op8 {
          i32x8 a[2];
          u32x4 r;
        };
        using KOp = typename std::conditional<FP8, Op8, bf16x8>::type;
        KOp kop[2][FP8 ? 1 : 9];
        // FP8: the scale of this lane's operand token per block (sct) as an E8M0 code (tokc:
        // its exponent field), and the scales of its weight tokens 16tb + 4g4 + e (scw), read
        // first so that their latency is spent here. They multiply exactly: a scale is a power
        // of two by the cache's contract.
        int tokc[2] = {127, 127};
        f32x4 scw[2];
        if constexpr (FP8) {
#pragma unroll
          for (int tb = 0; tb < 2; ++tb) {
            const float sct = *reinterpret_cast<const MLA_LDS float*>(kb + Tile8::BYTES +
                                                                      4 * (16 * tb + hl));
            tokc[tb] = (int)((__builtin_bit_cast(uint32_t, sct) >> 23) & 0xff);
            scw[tb] = *reinterpret_cast<const MLA_LDS f32x4*>(kb + Tile8::BYTES +
                                                              4 * (16 * tb + 4 * g4));
          }
        }
        auto read_half = [&](KOp* dst, int tb, int s0) {
          if constexpr (FP8) {
            const int h = s0 / 9;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
              const uint32_t o = 128 * (2 * h + i);
              const u32x4 p0 = *reinterpret_cast<const MLA_LDS u32x4*>(kb + ka8[tb][0] + o);
              const u32x4 p1 = *reinterpret_cast<const MLA_LDS u32x4*>(kb + ka8[tb][1] + o);
              dst[0].a[i] =
                  __builtin_bit_cast(i32x8, __builtin_shufflevector(p0, p1, 0, 1, 2, 3, 4, 5, 6, 7));
            }
            dst[0].r = *reinterpret_cast<const MLA_LDS u32x4*>(kb + kr8[tb][h]);
          } else {
#pragma unroll
            for (int i = 0; i < 9; ++i) {
              const int s = s0 + i;
              dst[i] = lds_read_b128(kb, ko[tb][s & 1] + 128 * (s >> 1));
            }
          }
        };
        auto mfma_half = [&](f32x4* c, const KOp* src, int s0, int tb) {
          if constexpr (FP8) {
            const int h = s0 / 9;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
              c[0] = mfma_scale_16x16x128_fp8(src[0].a[i], qh[2 * h + i], c[0], tokc[tb], qsc[0]);
              c[1] = mfma_scale_16x16x128_fp8(src[0].a[i], ql[2 * h + i], c[1], tokc[tb], qsc[1]);
            }
            c[h] = mfma_16x16x32(__builtin_bit_cast(bf16x8, src[0].r), qf[16 + h], c[h]);
          } else {
#pragma unroll
            for (int i = 0; i < 9; ++i) {
              const int s = s0 + i;
              c[s & 1] = mfma_16x16x32(src[i], qf[s], c[s & 1]);
            }
          }
        };
        static_assert(KST == 18, "two half-blocks of nine steps");
        const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
        f32x4 c0[2] = {zero4, zero4}, c1[2] = {zero4, zero4};
        read_half(kop[0], 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        read_half(kop[1], 0, 9);
        __builtin_amdgcn_sched_barrier(0);
        mfma_half(c0, kop[0], 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        read_half(kop[0], 1, 0);
        __builtin_amdgcn_sched_barrier(0);
        mfma_half(c0, kop[1], 9, 0);
        __builtin_amdgcn_sched_barrier(0);
        read_half(kop[1], 1, 9);
        __builtin_amdgcn_sched_barrier(0);
        mfma_half(c1, kop[0], 0, 1);
        __builtin_amdgcn_sched_barrier(0);
        // lane: head hl, tokens 16tb + 4g4 + e
        const int valid = min(kSub, ca.S - ca.j * kSub);
        const int pb = t & 1;
        MLA_LDS char* prow = (MLA_LDS char*)lds_p[pb] + (16 * a + hl) * PPITCH + 8 * g4;
        float v[2][4];
        auto scale_block = [&](int tb, const f32x4* c) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            v[tb][e] = 16 * tb + 4 * g4 + e < valid ? (c[0][e] + c[1][e]) * scale_log2 : -INFINITY;
        };
        float lsum = 0.f;
        auto weights_block = [&](int tb) {  // bf16 weights of block tb against m_ref, to P
          bf16x4 pv;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const __bf16 pbf = (__bf16)exp2f_fast(v[tb][e] - m_ref);
            // FP8: the weight that multiplies the unscaled values carries the token's scale
            // (exact: a power of two); l sums the weights themselves
            pv[e] = FP8 ? (__bf16)((float)pbf * scw[tb][e]) : pbf;
            lsum += (float)pbf;
          }
          *reinterpret_cast<MLA_LDS bf16x4*>(prow + 32 * tb) = pv;
        };
        if (!seg_first) {
          scale_block(0, c0);
          weights_block(0);
          mfma_half(c1, kop[1], 9, 1);
          constexpr int HALF_MFMA = FP8 ? 5 : 9, VALU_PER = FP8 ? 7 : 4;
#pragma unroll
          for (int i = 0; i < HALF_MFMA; ++i) {  // one MFMA, then some VALU work of block 0
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, VALU_PER, 0);
          }
          __builtin_amdgcn_sched_barrier(0);
          scale_block(1, c1);
          weights_block(1);
        } else {
          mfma_half(c1, kop[1], 9, 1);
          scale_block(0, c0);
          scale_block(1, c1);
        }
        float mx = -INFINITY;
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
          for (int e = 0; e < 4; ++e) mx = fmaxf(mx, v[tb][e]);
        mx = rows4_max(mx);  // over the head's 32 tokens (lanes hl, hl+16, hl+32, hl+48)
        float alpha = 1.f;
        int need = 0;
        if (seg_first) {
          m_ref = mx;
          l_lane = 0.f;
          weights_block(0);
          weights_block(1);
        } else if (mx > m_ref + kRescale) {  // rare: the head's reference max moves
          alpha = exp2f_fast(m_ref - mx);
          m_ref = mx;
          l_lane *= alpha;
          need = 1;
          lsum = 0.f;  // this tile's weights again, against the new reference
          weights_block(0);
          weights_block(1);
        }
        // the ballot is taken by the whole wave (inside a lane-0 branch it would see lane 0 only)
        const bool any_need = __ballot(need) != 0;
        if (lane == 0) lds_flag[pb][a] = any_need;
        if (g4 == 0) lds_alpha[pb][16 * a + hl] = alpha;
        l_lane += lsum;
        if (seg_last) {  // the head's row sum over the segment, its lse and 1/l
          const float lt = rows4_sum(l_lane);
          if (g4 == 0) {
            lds_invl[pb][16 * a + hl] = 1.f / lt;
            part_lse[(size_t)(ca.b + g) * H + head] = (m_ref + log2f_fast(lt)) * kLn2;
          }
        }
        cursor_next(ca, plan, seq_lens, B, max_pages, q_len);
      }
      block_sync_tagged<0>();
    }
  } else {
    // ================= value team: wave vw owns latent columns 128vw .. 128vw+127
    const int vw = wave - 4;
    const int t32 = lane & 31, hi = lane >> 5;
    const int G16 = lane >> 4, q16 = lane & 15;
    uint32_t dmo[TIPW];
#pragma unroll
    for (int k = 0; k < TIPW; ++k) dmo[k] = TileL::src_off(vw + 4 * k, lane, kSub);
    // value operand (transposing reads): rows 16ks + 8(G16/2) + 4hf + q16/4, latent columns
    // 128vw + 32nb + 16(G16%2) + 4(q16%4); column block nb >= 2 is 128 bytes further on
    uint32_t ov[2][2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int t = 8 * (G16 >> 1) + 4 * hf + (q16 >> 2);
        const int low = 4 * nb + 2 * (G16 & 1) + ((q16 >> 1) & 1);
        ov[hf][nb] = t * ROWB + 16 * (16 * vw + (low ^ Tile::swz(t))) + 8 * (q16 & 1);
      }
    // FP8 value operand (8-bit transposing reads): in each group of 16 lanes, lane w supplies
    // the 8 bytes at (token 16ks + 8(G16/2) + w/2, latent columns 128vw + 32nb + 16(G16%2) +
    // 8(w%2) ..+8), and lane l receives byte l%8 of the segments of lanes 2b + ((l >> 3) & 1),
    // b = 0..7: latent column 128vw + 32nb + (l & 31) of tokens 16ks + 8(l/32) + b
    uint32_t ov8[4];
    if constexpr (FP8) {
      const int t = 8 * (G16 >> 1) + (q16 >> 1);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        ov8[nb] = t * ROWB8 + 128 * vw + 16 * ((2 * nb + (G16 & 1)) ^ Tile8::swz(t)) +
                  8 * (q16 & 1);
    }
    const uint32_t pr = t32 * PPITCH + 16 * hi;  // P read: + 32*PPITCH*mb + 32*ks

    // tile loads. A loading wave keeps 64 page-table entries of the current sequence in one
    // VGPR (lane l: entry pw_base + l) and picks entries with readlane, so the loop issues no
    // scalar loads (the barrier would wait for them).
    Cursor lc = c0;
    int issued = 0;
    int pw_v = 0, pw_b = -1, pw_base = 0;
    // The next tile to load: its global base, valid rows and LDS buffer (lookup), then its
    // instructions (and, FP8, its scales), possibly in parts, then the cursor moves on
    // (advance).
    const char* nbase = kv;
    const float* nsc = kv_scales;  // FP8: the tile's 32 scales
    int nvalid = 0;
    MLA_LDS char* ndst = tiles;
    // FP8: lane l loads the scale of token min(l % 32, valid - 1) into byte 4l of the block
    auto sc_off = [&](int valid) { return 4u * (uint32_t)min(lane & 31, valid - 1); };
    auto set_scales = [&](int page, int j) {
      if constexpr (FP8) {
        page = page < 0 ? 0 : (page >= num_pages ? num_pages - 1 : page);
        nsc = kv_scales + (size_t)page * kPage + (j % Tile8::TPP) * kSub;
      }
    };
    auto lookup = [&]() {
      const int p = lc.j / Tile::TPP;
      if (lc.b != pw_b || p < pw_base || p >= pw_base + 64) {
        // refill: the load and its wait are one asm statement, so the compiler sees pw_v as
        // ready and puts no wait of its own before the readlane below (such a wait would drain
        // the tile loads in flight on every tile). Loads complete in order, so this wait also
        // lets the earlier tile loads land; it happens once per 64 pages or sequence.
        pw_b = lc.b;
        pw_base = p;
        const int idx = min(p + lane, max_pages - 1);
        const int32_t* src = page_table + (size_t)virt_row(lc.b, q_len) * max_pages + idx;
        asm volatile("global_load_dword %0, %1, off\n\ts_waitcnt vmcnt(0)"
                     : "=v"(pw_v) : "v"(src) : "memory");
      }
      const int page = __builtin_amdgcn_readlane(pw_v, p - pw_base);
      nbase = TileL::base_of(kv, page, lc.j, num_pages);
      set_scales(page, lc.j);
      nvalid = min(kSub, lc.S - lc.j * kSub);
      ndst = tiles + (issued % NBUF) * LB;
    };
    auto advance = [&]() {
      ++issued;
      cursor_next(lc, plan, seq_lens, B, max_pages, q_len);
    };
    auto issue_scales = [&]() {
      if constexpr (FP8) load_lds_4(nsc, sc_off(nvalid), ndst + Tile8::BYTES);
    };
    auto issue_next = [&]() {
      lookup();
      TileL::template issue<4>(nbase, nvalid, dmo, ndst, vw, lane);
      issue_scales();
      advance();
    };
    {
      // Tile 0 goes out at once with the page from the unit record. Beside it, the page window
      // of the sequence is loaded for the next tiles. The window load, tile 0's loads and the
      // wait for the window (loads complete in order: it is the oldest) form one asm
      // statement, so the window register is complete when the compiler first sees it and no
      // instruction can read it while the load is in flight (it is early-clobber: no input
      // shares its register). M0, the LDS destination, steps by 4 KiB per instruction.
      pw_b = lc.b;
      pw_base = lc.j / Tile::TPP;
      const int idx = pw_base + lane < max_pages ? pw_base + lane : max_pages - 1;
      const int32_t* src = page_table + (size_t)virt_row(lc.b, q_len) * max_pages + idx;
      nbase = TileL::base_of(kv, us.page, lc.j, num_pages);
      set_scales(us.page, lc.j);
      nvalid = min(kSub, lc.S - lc.j * kSub);
      ndst = tiles;
      uint32_t o[TIPW];
#pragma unroll
      for (int k = 0; k < TIPW; ++k)
        o[k] = nvalid >= kSub ? dmo[k] : TileL::src_off(vw + 4 * k, lane, nvalid);
      uint32_t m0 = (uint32_t)(uintptr_t)(ndst + vw * 1024);
      if constexpr (FP8) {
        // five tile loads, then the scales (M0 moved to the entry's scale block); the wait
        // leaves those six in flight
        static_assert(TIPW == 5 && IPW == 6, "five tile loads and one scale load per wave");
        const uint32_t m0_sc = (uint32_t)(uintptr_t)(ndst + Tile8::BYTES);
        asm volatile(
            "global_load_dword %0, %2, off\n\t"
            "global_load_lds_dwordx4 %4, %3\n\t"
            "s_add_u32 m0, m0, 0x1000\n\t"
            "global_load_lds_dwordx4 %5, %3\n\t"
            "s_add_u32 m0, m0, 0x1000\n\t"
            "global_load_lds_dwordx4 %6, %3\n\t"
            "s_add_u32 m0, m0, 0x1000\n\t"
            "global_load_lds_dwordx4 %7, %3\n\t"
            "s_add_u32 m0, m0, 0x1000\n\t"
            "global_load_lds_dwordx4 %8, %3\n\t"
            "s_mov_b32 m0, %11\n\t"
            "global_load_lds_dword %9, %10\n\t"
            "s_waitcnt vmcnt(6)"
            : "=&v"(pw_v), "+{m0}"(m0)
            : "v"(src), "s"(nbase), "v"(o[0]), "v"(o[1]), "v"(o[2]), "v"(o[3]), "v"(o[4]),
              "v"(sc_off(nvalid)), "s"(nsc), "s"(m0_sc)
            : "memory", "scc");
      } else {
      static_assert(IPW == 9, "nine loads per wave per tile");
      asm volatile(
          "global_load_dword %0, %2, off\n\t"
          "global_load_lds_dwordx4 %4, %3\n\t"
          "s_add_u32 m0, m0, 0x1000\n\t"
          "global_load_lds_dwordx4 %5, %3\n\t"
          "s_add_u32 m0, m0, 0x1000\n\t"
          "global_load_lds_dwordx4 %6, %3\n\t"
          "s_add_u32 m0, m0, 0x1000\n\t"
          "global_load_lds_dwordx4 %7, %3\n\t"
          "s_add_u32 m0, m0, 0x1000\n\t"
          "global_load_lds_dwordx4 %8, %3\n\t"
          "s_add_u32 m0, m0, 0x1000\n\t"
          "global_load_lds_dwordx4 %9, %3\n\t"
          "s_add_u32 m0, m0, 0x1000\n\t"
          "global_load_lds_dwordx4 %10, %3\n\t"
          "s_add_u32 m0, m0, 0x1000\n\t"
          "global_load_lds_dwordx4 %11, %3\n\t"
          "s_add_u32 m0, m0, 0x1000\n\t"
          "global_load_lds_dwordx4 %12, %3\n\t"
          "s_waitcnt vmcnt(9)"
          : "=&v"(pw_v), "+{m0}"(m0)
          : "v"(src), "s"(nbase), "v"(o[0]), "v"(o[1]), "v"(o[2]), "v"(o[3]), "v"(o[4]),
            "v"(o[5]), "v"(o[6]), "v"(o[7]), "v"(o[8])
          : "memory", "scc");
      }
      advance();
    }
    constexpr int MAXA = NBUF - 2;  // tiles in flight beyond the two in use
    while (issued < NBUF - 1 && issued < n) issue_next();
    wait_tiles<IPW, MAXA>(issued - 1);  // tile 0 landed
    block_sync_tagged<1>();

    // round -1: the score team works on tile 0
    if (1 < n) wait_tiles<IPW, MAXA>(issued - 2);  // tile 1 landed
    block_sync_tagged<1>();

    // global stores of one segment's partial per wave (both formats), counted in the tile wait
    // that follows them
    constexpr int kPartStores = 16;
    Cursor cb = c0;
    f32x16 acc[2][4];
    int r = 0;
    while (r < n) {  // one segment (a run of one sequence's tiles) per pass
      const int seg = min(cb.nj - cb.j, n - r);
      const int slot = cb.b + g;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = f32x16{};
      for (int k = 0; k < seg; ++k, ++r) {
        // tile r+NBUF-1 goes into the buffer tile r-1 left (read before the last barrier); its
        // loads are issued in three parts between the value MFMAs
        const bool load = issued < n;
        if (load) lookup();
        const int pb = r & 1;
        const MLA_LDS char* kb = tiles + (r % NBUF) * LB;
        const MLA_LDS char* pbuf = (const MLA_LDS char*)lds_p[pb];
        if (k > 0) {
          const u32x4 fl =
              *reinterpret_cast<const MLA_LDS u32x4*>((const MLA_LDS char*)lds_flag[pb]);
          if (fl[0] | fl[1] | fl[2] | fl[3]) {  // rare: some reference maxima moved
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) {
              const float a = lds_alpha[pb][32 * mb + t32];  // this lane's head
#pragma unroll
              for (int nb = 0; nb < 4; ++nb)
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[mb][nb][i] *= a;
            }
          }
        }
        // O^T[128 columns][64 heads] += V^T * P^T: the operand registers of P * V serve
        // unchanged with the roles swapped, and each lane then holds one head and four
        // consecutive columns (32nb + 8r4 + 4hi + e) per block
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          bf16x8 pa[2], vb[4];
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
            pa[mb] = lds_read_b128(pbuf, pr + 32 * PPITCH * mb + 32 * ks);
#pragma unroll
          for (int nb = 0; nb < 4; ++nb) {
            if constexpr (FP8) {
              typedef int v2i __attribute__((ext_vector_type(2)));
              const v2i w = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                  (MLA_LDS v2i*)(kb + ov8[nb] + ks * 16 * ROWB8));
              vb[nb] = cvt_fp8x8((uint32_t)w[0], (uint32_t)w[1], 1.0f);
            } else {
              vb[nb] = cat4(lds_read_tr16(kb, ov[0][nb & 1] + 128 * (nb >> 1) + ks * 16 * ROWB),
                            lds_read_tr16(kb, ov[1][nb & 1] + 128 * (nb >> 1) + ks * 16 * ROWB));
            }
          }
          if (load) {
            if constexpr (FP8) {
              if (ks == 0) Tile8::issue_part<4, 0, 2>(nbase, nvalid, dmo, ndst, vw, lane);
              else Tile8::issue_part<4, 2, 4>(nbase, nvalid, dmo, ndst, vw, lane);
            } else {
              if (ks == 0) Tile::issue_part<4, 0, 3>(nbase, nvalid, dmo, ndst, vw, lane);
              else Tile::issue_part<4, 3, 6>(nbase, nvalid, dmo, ndst, vw, lane);
            }
          }
#pragma unroll
          for (int nb = 0; nb < 4; ++nb)
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
              acc[mb][nb] = mfma_32x32x16(vb[nb], pa[mb], acc[mb][nb]);
        }
        if (load) {
          if constexpr (FP8) Tile8::issue_part<4, 4, 5>(nbase, nvalid, dmo, ndst, vw, lane);
          else Tile::issue_part<4, 6, 9>(nbase, nvalid, dmo, ndst, vw, lane);
          issue_scales();
          advance();
        }
        if (FP8 && k == seg - 1) {
          // Normalise and write this wave's block of the segment's partial, staged in the
          // bytes of tile r that only this wave read (its 128 FP8 columns of each 640-byte row,
          // 4 KiB): 32 heads x 64 columns per pass, head 32mb + t of the pass in row t, then
          // written as whole 128-byte rows (device scope). Within a row the 8-byte unit u sits
          // at u ^ 2((t >> 1) & 7): the 64 lanes of a write hit every bank twice, and 16-byte
          // pieces stay whole for the read-back.
          MLA_LDS char* stg = tiles + (r % NBUF) * LB + 128 * vw;
          int slot_e = slot, lane_e = lane;
          asm volatile("" : "+s"(slot_e), "+v"(lane_e));
          uint16_t* po = part_o + ((size_t)slot_e * H + HG * hh) * DC + 128 * vw;
          const int t32e = lane_e & 31;
          const int wsw = 2 * ((t32e >> 1) & 7);
#pragma unroll
          for (int mb = 0; mb < 2; ++mb) {
            const float il = lds_invl[pb][32 * mb + t32e];
#pragma unroll
            for (int half = 0; half < 2; ++half) {
#pragma unroll
              for (int nbl = 0; nbl < 2; ++nbl)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                  const f32x16& o = acc[mb][2 * half + nbl];
                  const int u = 8 * nbl + 2 * r4 + (lane_e >> 5);
                  const u32x2 w = {pack_bf16x2(o[4 * r4] * il, o[4 * r4 + 1] * il),
                                   pack_bf16x2(o[4 * r4 + 2] * il, o[4 * r4 + 3] * il)};
                  *reinterpret_cast<MLA_LDS u32x2*>(stg + t32e * ROWB8 + 8 * (u ^ wsw)) = w;
                }
              static_assert(2 * 2 * 4 == kPartStores, "stores per partial (mb, half, q4)");
#pragma unroll
              for (int q4 = 0; q4 < 4; ++q4) {  // 32 rows x 8 pieces of 16 bytes
                const int q = q4 * 64 + lane_e, row = q >> 3, piece = q & 7;
                const int rsw = 2 * ((row >> 1) & 7);
                store_16_device_scope(
                    po, 2 * ((32 * mb + row) * DC + 64 * half + piece * 8),
                    *reinterpret_cast<const MLA_LDS u32x4*>(stg + row * ROWB8 +
                                                            8 * ((2 * piece) ^ rsw)));
              }
            }
          }
        } else if (k == seg - 1) {
          // Normalise and write this wave's block of the segment's partial. It is staged, 32
          // heads at a time, in the bytes of tile r that only this wave read (256 bytes at
          // 256vw of each 1152-byte row), then written as whole 256-byte rows at device scope
          // (the combine reads them from other XCDs).
          MLA_LDS char* stg = tiles + (r % NBUF) * LB + 256 * vw;
          // (the slot and lane pass through empty asm so that the store addresses are formed
          // here, not kept in registers through the whole segment)
          int slot_e = slot, lane_e = lane;
          asm volatile("" : "+s"(slot_e), "+v"(lane_e));
          uint16_t* po = part_o + ((size_t)slot_e * H + HG * hh) * DC + 128 * vw;
          // Staging row t32 is head 32mb + t32; its 8-byte chunk c (four columns) sits at chunk
          // c ^ sw(row), sw(row) = 2((row >> 1) & 7), which spreads the 64 lanes of a write
          // over all banks (two per bank) and keeps 16-byte pieces whole for the read-back.
          const int t32e = lane_e & 31;
          const uint32_t wrow = t32e * ROWB + 8 * (lane_e >> 5);
          const int wsw = 2 * ((t32e >> 1) & 7);
#pragma unroll
          for (int mb = 0; mb < 2; ++mb) {
            const float il = lds_invl[pb][32 * mb + t32e];
#pragma unroll
            for (int nb = 0; nb < 4; ++nb)
#pragma unroll
              for (int r4 = 0; r4 < 4; ++r4) {
                const f32x16& o = acc[mb][nb];
                const uint32_t lo = pack_bf16x2(o[4 * r4] * il, o[4 * r4 + 1] * il);
                const uint32_t hi2 = pack_bf16x2(o[4 * r4 + 2] * il, o[4 * r4 + 3] * il);
                *reinterpret_cast<MLA_LDS uint64_t*>(stg + wrow + 8 * ((8 * nb + 2 * r4) ^ wsw)) =
                    (uint64_t)lo | ((uint64_t)hi2 << 32);
              }
            static_assert(2 * 8 == kPartStores, "stores per partial (mb, q8)");
#pragma unroll
            for (int q8 = 0; q8 < 8; ++q8) {  // 32 rows x 16 pieces of 16 bytes
              const int q = q8 * 64 + lane_e, row = q >> 4, piece = q & 15;
              const int rsw = 2 * ((row >> 1) & 7);
              store_16_device_scope(po, 2 * ((32 * mb + row) * DC + piece * 8),
                                    *reinterpret_cast<const MLA_LDS u32x4*>(
                                        stg + row * ROWB + 8 * ((2 * piece) ^ rsw)));
            }
          }
        }
        // tile r+2 landed (a wave that wrote a partial above has its stores behind the loads)
        if (r + 2 < n) {
          if (k == seg - 1) wait_tiles<IPW, MAXA, kPartStores>(issued - (r + 3));
          else wait_tiles<IPW, MAXA>(issued - (r + 3));
        }
        block_sync_tagged<1>();  // P of tile r+1 visible; tile r free
      }
      cb.j += seg - 1;
      cursor_next(cb, plan, seq_lens, B, max_pages, q_len);
    }
    wait_vmcnt<0>();
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
constexpr float kRescale = 64.f;  // log2 headroom before the running max must move
// FP8 cache: a token row is [c_KV as FP8 e4m3 (64 bytes) | k_R bf16 (16 bytes)], 80 bytes,
// and each token has an fp32 power-of-two scale in a separate array of the same page geometry.
// A loaded tile is its 5 KiB of rows followed by its 64 scales (256 bytes), in a three-deep
// ring (two in flight while one is used). The MFMA operands are formed from the FP8 bytes in
// registers: the score operand (8 latent values of one token row) is converted with that
// token's scale; the value operand (8 tokens of one latent column, from 8-bit transposing
// reads) is converted unscaled, and each token's scale multiplies its softmax weight instead.
// A power of two moves exactly between the two factors, so the products are those of the bf16
// cache holding c_KV * scale.
constexpr int ROWB8 = DC + 2 * DR;
using Tile8 = PagedTile<TT, ROWB8>;
constexpr int SB8 = Tile8::BYTES + 4 * TT;  // bytes of one loaded FP8 tile with its scales
// MXFP4 cache: a token row is [c_KV as E2M1 codes, two per byte, element 2k in the low nibble
// (32 bytes) | k_R bf16 (16 bytes)], 48 bytes, and each token has DC/32 = 2 E8M0 scale bytes
// (one per block of 32 latent elements) in a separate array of the same page geometry. A loaded
// tile is its 3 KiB of rows followed by its 128 scale bytes (in a 256-byte slot: the load moves
// 4 bytes a lane). The score operand (8 elements of one block of a token row) is converted with
// that block's scale. The value operand cannot carry the scale in the weight, as FP8 does: the
// scale changes along the latent dimension. So each tile's latent part is converted once, one
// token row per lane, into a bf16 copy in the wave's own LDS buffer, laid out as the bf16 tile,
// and the values are read from it as in the bf16 path.
constexpr int MXB = DC / 32;
constexpr int ROWB4 = DC / 2 + 2 * DR;
using Tile4 = PagedTile<TT, ROWB4>;
constexpr int SB4 = Tile4::BYTES + 256;  // bytes of one loaded MXFP4 tile with its scales
}  // namespace m2

// E8M0 scale byte -> the fp32 scale operand of the gfx950 scaled conversions: the byte as the
// exponent field (code 0 gives fp32 bits 0, which the conversions take as 2^-127, as E8M0 does;
// checked on the device)
__device__ __forceinline__ float e8m0_scale(uint32_t code) {
  return __builtin_bit_cast(float, code << 23);
}

// 8 E2M1 elements (the 4 bytes of w, element 2k in the low nibble of byte k) -> bf16, times sc
__device__ __forceinline__ bf16x8 cvt_fp4x8(uint32_t w, float sc) {
  const bf16x2 a0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0);
  const bf16x2 a1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1);
  const bf16x2 a2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2);
  const bf16x2 a3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3);
  return cat4(__builtin_shufflevector(a0, a1, 0, 1, 2, 3),
              __builtin_shufflevector(a2, a3, 0, 1, 2, 3));
}

// Waits until at most `after` (0..4) tiles of N load instructions each are still in flight.
template <int N>
__device__ __forceinline__ void wait_tiles_upto4(int after) {
  if (after >= 4) wait_vmcnt<4 * N>();
  else if (after == 3) wait_vmcnt<3 * N>();
  else if (after == 2) wait_vmcnt<2 * N>();
  else if (after == 1) wait_vmcnt<N>();
  else wait_vmcnt<0>();
}

template <int FMT, int NB>
__global__ void __launch_bounds__(256)
attn_mha2mla_kernel(const uint16_t* __restrict__ q_abs, const uint16_t* __restrict__ q_rope,
                    const char* __restrict__ kv, const int32_t* __restrict__ page_table,
                    const int32_t* __restrict__ seq_lens, int B, int max_pages, int q_len,
                    int num_pages,
                    const Plan* __restrict__ plan, int G, float scale_log2,
                    uint16_t* __restrict__ part_o, float* __restrict__ part_lse,
                    const void* __restrict__ kv_scales) {
  using namespace m2;
  constexpr bool FP8 = FMT == kKvFp8, MX = FMT == kKvMxfp4;
  using TileL = typename std::conditional<FP8, Tile8,
                typename std::conditional<MX, Tile4, Tile>::type>::type;  // the format as loaded
  constexpr int LB = FP8 ? SB8 : (MX ? SB4 : Tile::BYTES);  // bytes of one ring entry
  constexpr int IPW = TileL::INSTR + (FP8 || MX ? 1 : 0);   // load instructions per tile
  // MXFP4: the ring, then the bf16 copy of the current tile's latent part
  constexpr int WAVE_LDS = NB * LB + (MX ? Tile::BYTES : 0);
  // the plan for a quantised cache counts two work groups per CU (160 KiB of LDS)
  static_assert(FMT == kKvBf16 || kGroupsPerCuFp8 * kAttnWavesMha2Mla * WAVE_LDS <= 160 * 1024,
                "two work groups of a quantised cache must fit one CU's LDS");
  __shared__ __attribute__((aligned(1024))) char lds_tiles[kAttnWavesMha2Mla][WAVE_LDS];
  const float* sc8 = reinterpret_cast<const float*>(kv_scales);
  const unsigned char* sc4 = reinterpret_cast<const unsigned char*>(kv_scales);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform per wave
  const int g = blockIdx.x * kAttnWavesMha2Mla + wave;  // plan unit = wave
  const UnitStart us = load_unit(plan, B, g < G ? g : G - 1);
  const int n = g < G ? us.n : 0;  // tiles of this unit
  if (n <= 0) return;
  MLA_LDS char* tiles = (MLA_LDS char*)lds_tiles[wave];

  Cursor lc = {us.b, us.j, us.nj, us.S};
  Cursor cc = lc;
  uint32_t dmo[IPW];  // lane offsets of a full-tile load
#pragma unroll
  for (int k = 0; k < TileL::INSTR; ++k) dmo[k] = TileL::src_off(k, lane, TT);
  // The wave keeps 64 page-table entries of the current sequence in one VGPR (lane l: entry
  // pw_base + l) and picks them with readlane, so issuing a tile needs no scalar load (whose
  // wait would stall the wave before every tile). A refill is one asm statement, load and wait,
  // so the compiler adds no wait of its own before the readlane.
  int pw_v = 0, pw_b = -1, pw_base = 0;
  auto issue = [&](const Cursor& c, int buf) {
    const int p = c.j / Tile::TPP;
    if (c.b != pw_b || p < pw_base || p >= pw_base + 64) {
      pw_b = c.b;
      pw_base = p;
      const int idx = min(p + lane, max_pages - 1);
      const int32_t* src = page_table + (size_t)virt_row(c.b, q_len) * max_pages + idx;
      asm volatile("global_load_dword %0, %1, off\n\ts_waitcnt vmcnt(0)"
                   : "=v"(pw_v) : "v"(src) : "memory");
    }
    int page = __builtin_amdgcn_readlane(pw_v, p - pw_base);
    page = page < 0 ? 0 : (page >= num_pages ? num_pages - 1 : page);
    const int valid = min(TT, c.S - c.j * TT);
    MLA_LDS char* dst = tiles + buf * LB;
    TileL::template issue<1>(TileL::base_of(kv, page, c.j, num_pages), valid, dmo, dst, 0, lane);
    if constexpr (FP8)  // the tile's scales (slots past the end repeat the last valid one)
      load_lds_4(sc8 + (size_t)page * kPage + (c.j % Tile8::TPP) * TT,
                 4u * (uint32_t)min(lane, valid - 1), dst + Tile8::BYTES);
    if constexpr (MX)  // the page's 128 scale bytes, 4 a lane (lanes 32.. repeat the last 4)
      load_lds_4(sc4 + (size_t)page * kPage * MXB, 4u * (uint32_t)min(lane, TT * MXB / 4 - 1),
                 dst + Tile4::BYTES);
  };
  // FP8 -> bf16, 8 values from two words (bytes 0..7 in order), times 2^(exponent of sc)
  auto cvt8 = [](uint32_t w0, uint32_t w1, float sc) {
    const bf16x2 a0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, sc, false);
    const bf16x2 a1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, sc, true);
    const bf16x2 a2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, sc, false);
    const bf16x2 a3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, sc, true);
    return cat4(__builtin_shufflevector(a0, a1, 0, 1, 2, 3),
                __builtin_shufflevector(a2, a3, 0, 1, 2, 3));
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
  for (; issued < NB - 1 && issued < n; ++issued) {
    issue(lc, issued % NB);
    cursor_next(lc, plan, seq_lens, B, max_pages, q_len);
  }
  for (int it = 0; it < n; ++it) {
    if (seg_start) {
      start_segment(cc.b);
      seg_start = false;
    }
    wait_tiles_upto4<IPW>(issued - it - 1);  // tile it landed
    if (issued < n) {  // into the buffer of tile it-1, done with in the last pass
      issue(lc, issued % NB);
      cursor_next(lc, plan, seq_lens, B, max_pages, q_len);
      ++issued;
    }
    const MLA_LDS char* kb = tiles + (it % NB) * LB;
    const MLA_LDS float* ksc = reinterpret_cast<const MLA_LDS float*>(kb + Tile8::BYTES);
    const MLA_LDS unsigned char* ksc4 =
        reinterpret_cast<const MLA_LDS unsigned char*>(kb + Tile4::BYTES);
    const int valid = min(TT, cc.S - cc.j * TT);

    // ---- scores for tokens [32*mb2, 32*mb2 + 32)
    f32x16 s[2];
#pragma unroll
    for (int mb2 = 0; mb2 < 2; ++mb2) {
      const int row = 32 * mb2 + t32;
      f32x16 a = {};
      i16x4 kr;
      if constexpr (FP8) {  // latent values 16st + 8hi .. +8 of token row `row`, scaled
        const MLA_LDS char* rp = kb + row * ROWB8;
        const float sc = ksc[row];
#pragma unroll
        for (int st = 0; st < DC / 16; ++st) {
          const u32x2 w = *reinterpret_cast<const MLA_LDS u32x2*>(rp + 16 * st + 8 * hi);
          a = mfma_32x32x16(cvt8(w[0], w[1], sc), qf[st], a);
        }
        kr = *reinterpret_cast<const MLA_LDS i16x4*>(rp + DC + 8 * hi);
      } else if constexpr (MX) {  // elements 16st + 8hi .. +8 of token row `row`: block st / 2
        const MLA_LDS char* rp = kb + row * ROWB4;
        const float s0 = e8m0_scale(ksc4[MXB * row]), s1 = e8m0_scale(ksc4[MXB * row + 1]);
        static_assert(MXB == 2, "two latent blocks per token row");
#pragma unroll
        for (int st = 0; st < DC / 16; ++st) {
          const uint32_t w = *reinterpret_cast<const MLA_LDS uint32_t*>(rp + 8 * st + 4 * hi);
          a = mfma_32x32x16(cvt_fp4x8(w, st < 2 ? s0 : s1), qf[st], a);
        }
        kr = *reinterpret_cast<const MLA_LDS i16x4*>(rp + DC / 2 + 8 * hi);
      } else {
#pragma unroll
        for (int st = 0; st < DC / 16; ++st)
          a = mfma_32x32x16(lds_read_b128(kb, Tile::lds_off(row, 2 * st + hi)), qf[st], a);
        kr = *reinterpret_cast<const MLA_LDS i16x4*>(kb + Tile::lds_off(row, DC / 8) + 8 * hi);
      }
      s[mb2] = mfma_32x32x8(kr, qr4, a);
    }
    // ---- online softmax, lane = head t32 x 32 tokens
    // raw logits stay unscaled: the scale enters once in the tile maximum and as one FMA in
    // each exponent
    float mt = -INFINITY;
    if (valid == TT) {  // a full tile (all but a sequence's last): no tail mask
#pragma unroll
      for (int mb2 = 0; mb2 < 2; ++mb2)
#pragma unroll
        for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[mb2][r]);
    } else {
#pragma unroll
      for (int mb2 = 0; mb2 < 2; ++mb2)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int t = 32 * mb2 + 8 * (r >> 2) + 4 * hi + (r & 3);
          const float v = t < valid ? s[mb2][r] : -INFINITY;
          s[mb2][r] = v;
          mt = fmaxf(mt, v);
        }
    }
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64)) * scale_log2;
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
          const float p = exp2f_fast(__builtin_fmaf(s[mb2][8 * half + j], scale_log2, -m_used));
          if constexpr (FP8) {  // token 32mb2 + 16half + 8(j/4) + 4hi + j%4 carries its scale
            // the scale's power of two (its exponent bits), as the conversion applies it
            const float sc = __builtin_bit_cast(
                float, __builtin_bit_cast(uint32_t, ksc[32 * mb2 + 16 * half + 8 * (j >> 2) +
                                                        4 * hi + (j & 3)]) & 0x7F800000u);
            pa[2 * mb2 + half][j] = (__bf16)(p * sc);
          } else {
            pa[2 * mb2 + half][j] = (__bf16)p;
          }
          lsum += p;  // the unrounded weight: l differs from the sum of the bf16 weights by
                      // rounding noise of relative size 2^-9 / sqrt(tokens)
        }
    l_lane = l_lane * alpha + lsum;
    // MXFP4: this tile's latent part as bf16, token row `lane` per lane, into the wave's
    // buffer (rows past the end were loaded as copies of the last valid row; their scales
    // are taken from that row too, so that no slot outside the sequence is read)
    MLA_LDS char* vbuf = tiles + NB * LB;
    if constexpr (MX) {
      const int t = lane, ts = t < valid ? t : valid - 1;
      const float s0 = e8m0_scale(ksc4[MXB * ts]), s1 = e8m0_scale(ksc4[MXB * ts + 1]);
      const u32x4 w0 = *reinterpret_cast<const MLA_LDS u32x4*>(kb + t * ROWB4);
      const u32x4 w1 = *reinterpret_cast<const MLA_LDS u32x4*>(kb + t * ROWB4 + 16);
#pragma unroll
      for (int ch = 0; ch < DC / 8; ++ch)  // chunk ch: elements 8ch .. 8ch + 7, block ch / 4
        *reinterpret_cast<MLA_LDS bf16x8*>(vbuf + Tile::lds_off(t, ch)) =
            cvt_fp4x8(ch < 4 ? w0[ch] : w1[ch - 4], ch < 4 ? s0 : s1);
    }
    const MLA_LDS char* vb = MX ? vbuf : kb;  // where the bf16 values are read
    // ---- values: block kk holds, for lane half hi, the tokens
    //      32*mb2 + 16*half + 8*(j/4) + 4*hi + j%4  (j < 8), the order of the score layout
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int mb2 = kk >> 1, half = kk & 1;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        if constexpr (FP8) {
          // 8-bit transposing read: in each group of 16 lanes, lane w supplies the 8 bytes at
          // (token T(w >> 1), columns 32nb + 16(G16 & 1) + 8(w & 1) ..+8), and lane l receives
          // byte l % 8 of the segments of lanes 2b + ((l >> 3) & 1), b = 0..7: the column
          // 32nb + (l & 31) of the tokens T(b) = 32mb2 + 16half + 8(b/4) + 4hi + b%4
          const int w = q16, b = w >> 1;
          const int t = 32 * mb2 + 16 * half + 8 * (b >> 2) + 4 * (G16 >> 1) + (b & 3);
          typedef int v2i __attribute__((ext_vector_type(2)));
          const v2i r = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
              (MLA_LDS v2i*)(kb + t * ROWB8 + 32 * nb + 16 * (G16 & 1) + 8 * (w & 1)));
          acc[nb] = mfma_32x32x16(pa[kk], cvt8((uint32_t)r[0], (uint32_t)r[1], 1.0f), acc[nb]);
          continue;
        }
        bf16x4 v2[2];
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          const int t = 32 * mb2 + 16 * half + 8 * p + 4 * (G16 >> 1) + (q16 >> 2);
          const int c0 = 32 * nb + 16 * (G16 & 1) + 4 * (q16 & 3);
          v2[p] = lds_read_tr16(vb, Tile::lds_off(t, c0 >> 3) + (c0 & 7) * 2);
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
          store_2_device_scope(po, 2 * (h * DC + 32 * nb + t32),
                               bf16_bits((__bf16)(acc[nb][r] * ih)));
      }
      seg_start = true;
    }
    cursor_next(cc, plan, seq_lens, B, max_pages, q_len);
  }
}

hipError_t launch_attention(int shape, const void* q_abs, const void* q_rope, const void* kv,
                            const int32_t* page_table, const int32_t* seq_lens, int B,
                            int max_pages, int q_len, int num_pages, const void* plan, int G,
                            float scale_log2, void* part_o, float* part_lse,
                            const void* kv_scales, int kv_format, const Launch& L) {
  if (shape == kShapeDeepSeek) {
    // two head halves per tile stream, paired 8 ids apart; ids padded to whole groups of 16
    const int blocks = 16 * ((G + 7) / 8);
    auto go = [&](auto kernel) {
      return launch_kernel(kernel, dim3(blocks), dim3(64 * ds::NW), L, (const uint16_t*)q_abs,
                           (const uint16_t*)q_rope, (const char*)kv, page_table, seq_lens, B,
                           max_pages, q_len, num_pages, (const Plan*)plan, G, scale_log2,
                           (uint16_t*)part_o, part_lse, (const float*)kv_scales);
    };
    if (kv_format == kKvMxfp4) return hipErrorInvalidValue;  // not built at these widths
    return kv_format == kKvFp8 ? go(attn_deepseek_kernel<true>) : go(attn_deepseek_kernel<false>);
  }
  const int blocks = (G + kAttnWavesMha2Mla - 1) / kAttnWavesMha2Mla;
  auto go = [&](auto kernel) {
    return launch_kernel(kernel, dim3(blocks), dim3(64 * kAttnWavesMha2Mla), L,
                         (const uint16_t*)q_abs, (const uint16_t*)q_rope, (const char*)kv,
                         page_table, seq_lens, B, max_pages, q_len, num_pages,
                         (const Plan*)plan, G, scale_log2, (uint16_t*)part_o, part_lse,
                         kv_scales);
  };
  // FP8: a three-deep ring of 5.25 KiB tiles (16 KiB a wave) lets two work groups share a
  // CU, two waves a SIMD; MXFP4: a three-deep ring of 3.25 KiB tiles and the 9 KiB bf16 copy
  // (18.75 KiB a wave), also two work groups a CU
  if (kv_format == kKvFp8) return go(attn_mha2mla_kernel<kKvFp8, kRingFp8>);
  if (kv_format == kKvMxfp4) return go(attn_mha2mla_kernel<kKvMxfp4, kRingFp8>);
  return go(attn_mha2mla_kernel<kKvBf16, m2::NBUF>);
}

}  // namespace mla
