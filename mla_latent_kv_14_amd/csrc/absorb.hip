// K1: absorbed query, q_abs[b,h,c] = sum_d q_nope[b,h,d] * W_UK[h,d,c]
// (lpnh.cn/news/2494972 S2.1: W_uk folds into the query side; bhfrc.com/news/60867 S4 path B).
//
// One work group per (head h, block of CB latent columns). The W_UK block [d_n x CB] is copied
// to LDS with direct global->LDS loads (32-byte units XOR-swizzled by row so that the
// transposing reads of four consecutive rows hit distinct banks), then
//   q_abs^T[c, b] = W_UK[h]^T[c, d] * q_nope^T[d, b]
// runs on 16x16x32 bf16 MFMA: the W operand comes from transposing LDS reads, the q_nope operand
// straight from global memory (8 consecutive d per lane), fp32 accumulation, bf16 (RNE) out.
// The kernel streams 2*H*d_n*d_c bytes of weight once; it is HBM-bound.
//
// Extra blocks (the first ones, so that they are dispatched at once: their chain of dependent
// loads is the longest in the kernel) write the work plan for the attention kernel (see Plan in
// device.h), in parallel with the others. Each plan block redoes the prefix sum over the
// sequences (cheap up to a few thousand) and resolves every thread's share of the units, at
// most one unit per thread where the block count allows: a unit costs a search, a dependent
// page-table load and a store, and a second round of them a few microseconds.
#include "device.h"
#include "kernels.h"

namespace mla {

// off[b] = sum_{b' < b} ceil(S_b' / TT) with S clamped; header {total, per, groups}; and the
// start record of every unit (see UnitStart).
// Batches up to this size keep offsets and lengths in LDS (the scratch passed in).
constexpr int kSeqInLds = 4096;
constexpr int kPlanLdsBytes = (2 * kSeqInLds + 8) * 4;

__device__ void build_plan(const int32_t* __restrict__ seq_lens,
                           const int32_t* __restrict__ page_table, int B, int max_pages,
                           int q_len, int G, int TT, Plan* __restrict__ plan,
                           MLA_LDS char* scratch, int part, int parts) {
  MLA_LDS int32_t* seq_off = (MLA_LDS int32_t*)scratch;
  MLA_LDS int32_t* seq_len = seq_off + kSeqInLds;
  MLA_LDS int32_t* wave_tot = seq_len + kSeqInLds;
  MLA_LDS int32_t& carry = wave_tot[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) carry = 0;
  __syncthreads();
  int32_t* off = plan_off(plan);
  for (int base = 0; base < B; base += 256) {
    const int b = base + tid;
    int n = 0, S = 0;
    if (b < B) {
      S = virt_len(clamp_len(seq_lens[virt_row(b, q_len)], max_pages), b, q_len);
      n = (S + TT - 1) / TT;
    }
    int x = n;  // inclusive wave scan
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      int y = __shfl_up(x, d, 64);
      if (lane >= d) x += y;
    }
    if (lane == 63) wave_tot[wave] = x;
    __syncthreads();
    int before = carry;
    for (int w = 0; w < wave; ++w) before += wave_tot[w];
    if (b < B) {
      if (part == 0) off[b] = before + x - n;
      if (b < kSeqInLds) {
        seq_off[b] = before + x - n;
        seq_len[b] = S;
      }
    }
    __syncthreads();
    if (tid == 0) carry += wave_tot[0] + wave_tot[1] + wave_tot[2] + wave_tot[3];
    __syncthreads();
  }
  const int g = G < 1 ? 1 : G;
  const int total = carry;
  const int per = (total + g - 1) / g;
  if (tid == 0 && part == 0) {
    plan->total = total;
    plan->per = per;
    plan->groups = g;
    plan->pad = 0;
  }
  UnitStart* start = plan_units(plan, B);
  auto write_unit = [&](int u, int b, int j, int S, int page) {
    UnitStart rec;
    rec.b = b;
    rec.j = j;
    rec.nj = (S + TT - 1) / TT;
    rec.S = S;
    rec.page = page;
    rec.n = min(per, total - u * per);
    rec.pad[0] = rec.pad[1] = 0;
    start[u] = rec;
  };
  // idle units (no tiles: u * per >= total) get an all-zero record
  for (int u = part * 256 + tid; u < g; u += parts * 256)
    if ((long long)u * per >= total) start[u] = UnitStart{0, 0, 0, 0, 0, 0, {0, 0}};
  if (B <= kSeqInLds) {
    // every unit on its own: its sequence by binary search over the offsets in LDS (the last
    // b with off[b] <= u*per; sequences with no tiles share their successor's offset and are
    // skipped by taking the last), then the page of its first tile
    for (int u0 = part * 256 + tid; u0 < g; u0 += 4 * 256 * parts) {
      int ub[4], uj[4], page[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int u = u0 + k * 256 * parts;
        ub[k] = -1;
        uj[k] = 0;
        page[k] = 0;
        if (u < g && (long long)u * per < total) {
          const int t = u * per;
          int lo = 0, hi = B - 1;
          while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (seq_off[mid] <= t) lo = mid; else hi = mid - 1;
          }
          ub[k] = lo;
          uj[k] = t - seq_off[lo];
          page[k] = page_table[(size_t)virt_row(lo, q_len) * max_pages + (uj[k] * TT) / kPage];
        }
      }
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (ub[k] >= 0)
          write_unit(u0 + k * 256 * parts, ub[k], uj[k], seq_len[ub[k]], page[k]);
    }
  } else if (part == 0) {  // (one plan block for large batches)
    // large batches: each thread walks the units that start in its sequences
    for (int b = tid; b < B; b += 256) {
      const int S = virt_len(clamp_len(seq_lens[virt_row(b, q_len)], max_pages), b, q_len);
      const int n = (S + TT - 1) / TT;
      const int o = off[b];
      for (int u = (o + per - 1) / per; u < g && (long long)u * per < o + n; ++u) {
        const int j = u * per - o;
        write_unit(u, b, j, S,
                   page_table[(size_t)virt_row(b, q_len) * max_pages + (j * TT) / kPage]);
      }
    }
  }
}

template <int DN, int DC, int CB>
__global__ __launch_bounds__(256) void absorb_kernel(const uint16_t* __restrict__ q_nope,
                                                     const uint16_t* __restrict__ W_UK,
                                                     uint16_t* __restrict__ q_abs, int B, int H,
                                                     const int32_t* __restrict__ seq_lens,
                                                     const int32_t* __restrict__ page_table,
                                                     int max_pages, int q_len, int G, int TT,
                                                     Plan* plan, int plan_blocks) {
  constexpr int DNP = (DN + 31) / 32 * 32;  // contraction padded to the MFMA K of 32
  constexpr int ROWB = CB * 2;              // LDS bytes per W row
  constexpr int UNITS = ROWB / 32;          // 32-byte units per row (swizzle period)
  constexpr int NCHUNK = DN * ROWB / 16;    // 16-byte pieces of the W block
  static_assert(NCHUNK % 64 == 0, "W block must be whole KiB");
  static_assert(DN % 8 == 0 && CB % 16 == 0 && DC % CB == 0, "shape");
  // the W block, or in the plan block the plan builder's scratch
  constexpr int LDS_BYTES = DNP * ROWB > kPlanLdsBytes ? DNP * ROWB : kPlanLdsBytes;
  __shared__ __attribute__((aligned(16))) char wt[LDS_BYTES];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nblk = DC / CB;
  if (blockIdx.x < plan_blocks) {  // the first blocks write the work plan, nothing else
    build_plan(seq_lens, page_table, B, max_pages, q_len, G, TT, plan, (MLA_LDS char*)wt,
               blockIdx.x, plan_blocks);
    return;
  }
  const int h = (blockIdx.x - plan_blocks) / nblk, cblk = (blockIdx.x - plan_blocks) % nblk;

  // ---- stage W_UK[h][0:DN][cblk*CB : +CB] in LDS
  const char* Wg = reinterpret_cast<const char*>(W_UK + (size_t)h * DN * DC + (size_t)cblk * CB);
  MLA_LDS char* wl = (MLA_LDS char*)wt;
  for (int k = wave; k < NCHUNK / 64; k += 4) {
    const int q = k * 64 + lane;
    const int row = q / (ROWB / 16), p = q % (ROWB / 16);
    const int lunit = (p >> 1) ^ (row % UNITS);
    load_lds_16(Wg, (uint32_t)(row * DC * 2 + lunit * 32 + (p & 1) * 16), wl + k * 1024);
  }
  for (int i = DN * ROWB / 16 + tid; i < DNP * ROWB / 16; i += 256)  // zero pad rows
    *reinterpret_cast<MLA_LDS u32x4*>(wl + i * 16) = u32x4{0, 0, 0, 0};

  // ---- q_abs^T block [CB x B] = W^T [CB x DNP] * q_nope^T [DNP x B]. Wave w takes sequence
  // block nb and the m-blocks w, w+4, ...; its q_nope operand is loaded while W is in flight.
  const int G16 = lane >> 4, q16 = lane & 15;
  constexpr int KS = DNP / 32;
  constexpr int MBLK = CB / 16;
  const int nblocks = (B + 15) / 16;
  const uint16_t* qn = q_nope + (size_t)h * DN;
  auto load_q = [&](int nb, bf16x8* bq) {
    // unconditional loads from clamped (in-bounds) addresses, zeroed afterwards where the
    // sequence or the contraction index lies past the end
    const int b = nb * 16 + q16, bc = b < B ? b : B - 1;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int d0 = ks * 32 + 8 * G16, dc = d0 < DN ? d0 : DN - 8;
      const u32x4 raw = *reinterpret_cast<const u32x4*>(qn + (size_t)bc * H * DN + dc);
      const uint32_t keep = (b < B && d0 < DN) ? 0xffffffffu : 0u;
      bq[ks] = __builtin_bit_cast(bf16x8, raw & keep);
    }
  };
  // up to QB sequence blocks of q_nope are loaded at a time, all in flight together (the first
  // ones while W is in flight)
  constexpr int QB = 4;
  bf16x8 bq[QB][KS];
#pragma unroll
  for (int i = 0; i < QB; ++i)
    if (i < nblocks) {
      load_q(i, bq[i]);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) settle(bq[i][ks]);
    }
  wait_vmcnt<0>();
  __syncthreads();

  for (int nb0 = 0; nb0 < nblocks; nb0 += QB) {
    if (nb0 > 0) {
#pragma unroll
      for (int i = 0; i < QB; ++i)
        if (nb0 + i < nblocks) load_q(nb0 + i, bq[i]);
    }
#pragma unroll
    for (int i = 0; i < QB; ++i) {
    const int nb = nb0 + i;
    if (nb >= nblocks) break;
    const int b = nb * 16 + q16;
    for (int mb = wave; mb < MBLK; mb += 4) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int row0 = ks * 32 + 8 * G16 + (q16 >> 2);
        const int row1 = row0 + 4;
        const uint32_t o0 = row0 * ROWB + ((mb ^ (row0 % UNITS)) * 32) + 8 * (q16 & 3);
        const uint32_t o1 = row1 * ROWB + ((mb ^ (row1 % UNITS)) * 32) + 8 * (q16 & 3);
        acc = mfma_16x16x32(cat4(lds_read_tr16(wl, o0), lds_read_tr16(wl, o1)), bq[i][ks], acc);
      }
      if (b < B) {
        const int c0 = cblk * CB + mb * 16 + 4 * G16;
        bf16x4 o = {(__bf16)acc[0], (__bf16)acc[1], (__bf16)acc[2], (__bf16)acc[3]};
        *reinterpret_cast<bf16x4*>(q_abs + ((size_t)b * H + h) * DC + c0) = o;
      }
    }
    }
  }
}

hipError_t launch_absorb(int shape, const void* q_nope, const void* W_UK, void* q_abs, int B,
                         int H, const int32_t* seq_lens, const int32_t* page_table, int max_pages,
                         int q_len, int G, void* plan, const Launch& L) {
  // plan blocks: one per 256 units (up to 8) while the offsets fit in LDS, else one
  const int PB = B <= kSeqInLds ? min(8, max(1, (G + 255) / 256)) : 1;
  if (shape == kShapeDeepSeek) {
    constexpr int DN = 128, DC = 512, CB = 128;
    return launch_kernel(absorb_kernel<DN, DC, CB>, dim3(H * (DC / CB) + PB), dim3(256), L,
                         (const uint16_t*)q_nope, (const uint16_t*)W_UK, (uint16_t*)q_abs, B, H,
                         seq_lens, page_table, max_pages, q_len, G, (int)kSub, (Plan*)plan, PB);
  }
  constexpr int DN = 120, DC = 64, CB = 64;
  return launch_kernel(absorb_kernel<DN, DC, CB>, dim3(H * (DC / CB) + PB), dim3(256), L,
                       (const uint16_t*)q_nope, (const uint16_t*)W_UK, (uint16_t*)q_abs, B, H,
                       seq_lens, page_table, max_pages, q_len, G, (int)kPage, (Plan*)plan, PB);
}

}  // namespace mla
