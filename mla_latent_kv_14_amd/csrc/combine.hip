// K3: merge the split partials of each sequence and up-project through W_UV.
//
//   lse_b      = ln sum_s exp(lse_s)                       over the segments s of sequence b
//   o_lat[c]   = sum_s exp(lse_s - lse_b) * o_s[c]         (fp32; o_s are normalised partials)
//   out[b,h,e] = sum_c o_lat[c] * W_UV[h,c,e]              (lpnh.cn/news/2494972 S2.1, v = c_kv W_uv)
//
// One work group per (head h, group of 16 sequences, block of EB output columns). With EB = 64
// the two halves of a (head, group) get block ids 8 apart, which places them on the same XCD:
// the second read of the partials hits its L2. At the DeepSeek widths EB = d_v = 128 (a head's
// partials are read by one work group) when there are enough (head, group) pairs to fill the
// chip, else EB = 64 (twice the work groups, half of W_UV each); at the MHA2MLA widths (small
// W_UV) EB = 64.
//
// The W_UV block [d_latent x EB] goes to LDS by direct loads (32-byte units XOR-swizzled by
// row) and stays in flight while the partials are merged. For the merge every thread owns one
// 16-byte column chunk of a sequence's latent row (or 1/J of its slots, when the rows are
// short); it issues the loads of all its slots (rows and their lse values) at once, forms the
// merged lse from the values it holds, and sums the weighted rows in fp32. The merged rows are
// rounded once to bf16 in LDS, then out^T[e, b] = W^T[e, c] * o_lat^T[c, b] runs on 16x16x32
// bf16 MFMA with transposing reads for the W operand. A sequence with no tokens gets out = 0
// and lse = -inf.
#include "device.h"
#include "kernels.h"

namespace mla {

namespace comb {
constexpr int NT = 1024;  // threads per work group
constexpr int SEQ = 16;   // sequences per work group (the MFMA N)
constexpr int CAP = 8;    // slots per thread whose loads are issued together
// At the DeepSeek widths, from this many (head, group) pairs on, a work group takes all 128
// output columns of its head (below it, two work groups of 64 columns fill more of the chip).
constexpr int kWholeHeadGroups = 256;
}  // namespace comb

// LAT: write the merged latent rows o_lat [B][H][DC] (bf16) to `out` instead of applying W_UV
// (the output projection then runs as a separate product with a merged weight).
template <int H, int DC, int DV, int EB, bool LAT = false>
__global__ void __launch_bounds__(comb::NT)
combine_kernel(const uint16_t* __restrict__ part_o, const float* __restrict__ part_lse,
               const Plan* __restrict__ plan, const uint16_t* __restrict__ W_UV,
               uint16_t* __restrict__ out, float* __restrict__ lse_out, int B, int groups) {
  using namespace comb;
  constexpr int ROWB = EB * 2;        // LDS bytes per W row
  constexpr int UNITS = ROWB / 32;    // swizzle period (32-byte units per row)
  constexpr int NCHUNK = DC * ROWB / 16;
  constexpr int OPITCH = DC * 2 + 16; // bytes per merged latent row in LDS
  constexpr int NCH = DC / 8;         // 16-byte chunks of a latent row
  constexpr int ITEMS = SEQ * NCH;    // (sequence, chunk) items of a work group
  constexpr int J = ITEMS >= NT ? 1 : NT / ITEMS;  // threads sharing one item (split by slot)
  constexpr int IPT = ITEMS >= NT ? ITEMS / NT : 1; // items per thread
  constexpr int NEB = DV / EB;  // column blocks per head: 1, or 2 (paired 8 ids apart)
  static_assert(NEB * EB == DV && (NEB == 1 || NEB == 2), "column blocks");
  static_assert(NCHUNK % 64 == 0 && DC % 32 == 0, "shape");
  static_assert(ITEMS * J == NT * IPT && (J & (J - 1)) == 0 && J <= 64, "item split");
  __shared__ __attribute__((aligned(16))) char lds_w[DC * ROWB];
  __shared__ __attribute__((aligned(16))) char lds_o[SEQ * OPITCH];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int x = blockIdx.x;
  const int eblk = NEB == 2 ? (x >> 3) & 1 : 0;
  const int grp = NEB == 2 ? ((x >> 4) << 3) | (x & 7) : x;  // (sequence group, head)
  if (grp >= groups) return;                  // padding block: leaves before any barrier
  const int h = grp % H, b0 = (grp / H) * SEQ;
  MLA_LDS char* wl = (MLA_LDS char*)lds_w;
  MLA_LDS char* ol = (MLA_LDS char*)lds_o;

  // ---- stage W_UV[h][:, eblk*EB : +EB] (completes during the merge)
  const char* Wg = reinterpret_cast<const char*>(W_UV + (size_t)h * DC * DV + (size_t)eblk * EB);
  if (!LAT)
  for (int k = wave; k < NCHUNK / 64; k += NT / 64) {
    const int q = k * 64 + lane;
    const int row = q / (ROWB / 16), p = q % (ROWB / 16);
    const int lunit = (p >> 1) ^ (row % UNITS);
    load_lds_16(Wg, (uint32_t)(row * DV * 2 + lunit * 32 + (p & 1) * 16), wl + k * 1024);
  }

  // ---- merge. The plan is read with scalar loads (lane l of every wave gets sequence b0+l's
  // first slot and slot count), so that waiting for it never waits for the W block.
  const int total = ld_uniform(&plan->total), per = ld_uniform(&plan->per);
  const int32_t* off = plan_off(plan);
  int offv = total;
#pragma unroll
  for (int l = 0; l <= SEQ; ++l) {  // lane SEQ: first tile after the group
    const int b = b0 + l;
    const int val = b < B ? ld_uniform(off + b) : total;
    offv = lane == l ? val : offv;
  }
  const int offn = __shfl_down(offv, 1, 64);  // first tile of the next sequence
  int firstv = 0, countv = 0;
  if (lane < SEQ && b0 + lane < B) {
    const int nt = offn - offv;
    if (nt > 0) {
      const int g0 = offv / per, g1 = (offv + nt - 1) / per;
      firstv = g0 + b0 + lane;
      countv = g1 - g0 + 1;
    }
  }
  const int j = tid % J;
  const size_t slot_stride = (size_t)H * DC;  // elements between consecutive slots of a head
  int first[IPT], count[IPT];
  bf16x8 v[IPT][CAP];
  float ls[IPT][CAP];
#pragma unroll
  for (int it = 0; it < IPT; ++it) {
    const int item = tid / J + it * (NT / J);
    const int bi = item / NCH, ch = item % NCH;
    first[it] = __shfl(firstv, bi, 64);
    count[it] = __shfl(countv, bi, 64);
    const uint16_t* src = part_o + ((size_t)first[it] * H + h) * DC + ch * 8;
    const float* lsrc = part_lse + (size_t)first[it] * H + h;
    // Unconditional loads (no branches between them, so none waits for another): a slot past
    // the sequence's last one re-reads that last slot, and its lse is replaced by -inf, which
    // gives it weight 0. With no slot at all (count 0) nothing loaded is used.
    const int last = count[it] > 0 ? count[it] - 1 : 0;
#pragma unroll
    for (int u = 0; u < CAP; ++u) {
      const int s = j + J * u;
      const int sc = s < last ? s : last;
      v[it][u] = *reinterpret_cast<const bf16x8*>(src + (size_t)sc * slot_stride);
      const float l = lsrc[(size_t)sc * H];
      ls[it][u] = s < count[it] ? l : -INFINITY;
    }
  }
  int lse_at[IPT];  // lse_out index of this thread's item, or -1
  float lse_val[IPT];
#pragma unroll
  for (int it = 0; it < IPT; ++it) {
    lse_at[it] = -1;
    lse_val[it] = 0.f;
  }
#pragma unroll
  for (int it = 0; it < IPT; ++it) {
    const int item = tid / J + it * (NT / J);
    const int bi = item / NCH, ch = item % NCH, b = b0 + bi;
    const int cnt = count[it];
    const float* lsrc = part_lse + (size_t)first[it] * H + h;
    // merged lse: max, then sum of exponentials, over all slots of the sequence
    // Slots past the first J*CAP (a sequence spread over many units) are taken TB at a time,
    // each batch's loads issued together (clamped to the last slot, masked by the count).
    constexpr int TB = 8;
    float m = -INFINITY;
#pragma unroll
    for (int u = 0; u < CAP; ++u) m = fmaxf(m, ls[it][u]);
    for (int s0 = j + J * CAP; s0 < cnt; s0 += J * TB) {
      float l[TB];
#pragma unroll
      for (int u = 0; u < TB; ++u) l[u] = lsrc[(size_t)min(s0 + J * u, cnt - 1) * H];
#pragma unroll
      for (int u = 0; u < TB; ++u) m = fmaxf(m, l[u]);  // clamped copies repeat a real value
    }
#pragma unroll
    for (int d = 1; d < J; d <<= 1) m = fmaxf(m, __shfl_xor(m, d, 64));
    float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float L = -INFINITY;
    if (cnt > 0) {
      float z = 0.f;
#pragma unroll
      for (int u = 0; u < CAP; ++u) z += __expf(ls[it][u] - m);  // exp(-inf) = 0 past count
      for (int s0 = j + J * CAP; s0 < cnt; s0 += J * TB) {
        float l[TB];
#pragma unroll
        for (int u = 0; u < TB; ++u) l[u] = lsrc[(size_t)min(s0 + J * u, cnt - 1) * H];
#pragma unroll
        for (int u = 0; u < TB; ++u) z += s0 + J * u < cnt ? __expf(l[u] - m) : 0.f;
      }
#pragma unroll
      for (int d = 1; d < J; d <<= 1) z += __shfl_xor(z, d, 64);
      L = m + __logf(z);
#pragma unroll
      for (int u = 0; u < CAP; ++u) {
        const float w = __expf(ls[it][u] - L);
#pragma unroll
        for (int e = 0; e < 8; ++e) a[e] += w * (float)v[it][u][e];
      }
      const uint16_t* src = part_o + ((size_t)first[it] * H + h) * DC + ch * 8;
      for (int s0 = j + J * CAP; s0 < cnt; s0 += J * TB) {
        float l[TB];
        bf16x8 r[TB];
#pragma unroll
        for (int u = 0; u < TB; ++u) {
          const int sc = min(s0 + J * u, cnt - 1);
          l[u] = lsrc[(size_t)sc * H];
          r[u] = *reinterpret_cast<const bf16x8*>(src + (size_t)sc * slot_stride);
        }
#pragma unroll
        for (int u = 0; u < TB; ++u) {
          const float w = s0 + J * u < cnt ? __expf(l[u] - L) : 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) a[e] += w * (float)r[u][e];
        }
      }
    }
#pragma unroll
    for (int d = 1; d < J; d <<= 1)
#pragma unroll
      for (int e = 0; e < 8; ++e) a[e] += __shfl_xor(a[e], d, 64);
    if (j == 0) {
      bf16x8 o;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = (__bf16)a[e];
      if (LAT) {
        if (b < B) *reinterpret_cast<bf16x8*>(out + ((size_t)b * H + h) * DC + ch * 8) = o;
      } else {
        *reinterpret_cast<MLA_LDS bf16x8*>(ol + bi * OPITCH + ch * 16) = o;
      }
      if (ch == 0 && eblk == 0 && b < B && lse_out) {
        // stored at the very end (a store counts like a load in the wait for the W block,
        // and would hold every wave at that wait for its write latency)
        if (LAT) lse_out[(size_t)b * H + h] = L;
        lse_at[it] = (int)((size_t)b * H + h);
        lse_val[it] = L;
      }
    }
  }
  if (LAT) return;
  wait_vmcnt<0>();  // W block
  block_sync();

  // ---- out^T[e][b]: waves 0..3 take 16 columns e each
  if (wave < EB / 16) {
    const int G16 = lane >> 4, q16 = lane & 15;
    const int mb = wave;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int ks = 0; ks < DC / 32; ++ks) {
      const int row0 = ks * 32 + 8 * G16 + (q16 >> 2), row1 = row0 + 4;
      const bf16x4 a0 = lds_read_tr16(wl, row0 * ROWB + ((mb ^ (row0 % UNITS)) * 32) + 8 * (q16 & 3));
      const bf16x4 a1 = lds_read_tr16(wl, row1 * ROWB + ((mb ^ (row1 % UNITS)) * 32) + 8 * (q16 & 3));
      const bf16x8 bo = lds_read_b128(ol, q16 * OPITCH + (ks * 32 + 8 * G16) * 2);
      acc = mfma_16x16x32(cat4(a0, a1), bo, acc);
    }
    const int b = b0 + q16;
    if (b < B) {
      const int e0 = eblk * EB + mb * 16 + 4 * G16;
      bf16x4 o = {(__bf16)acc[0], (__bf16)acc[1], (__bf16)acc[2], (__bf16)acc[3]};
      *reinterpret_cast<bf16x4*>(out + ((size_t)b * H + h) * DV + e0) = o;
    }
  }
#pragma unroll
  for (int it = 0; it < IPT; ++it)
    if (lse_at[it] >= 0) lse_out[lse_at[it]] = lse_val[it];
}

hipError_t launch_combine_latent(int shape, const void* part_o, const float* part_lse,
                                 const void* plan, void* o_lat, float* lse_out, int B, int H,
                                 const Launch& L) {
  const int groups = H * ((B + comb::SEQ - 1) / comb::SEQ);
  const uint16_t* po = (const uint16_t*)part_o;
  const Plan* pl = (const Plan*)plan;
  uint16_t* o = (uint16_t*)o_lat;
  if (shape == kShapeDeepSeek)
    return launch_kernel(combine_kernel<128, 512, 128, 128, true>, dim3(groups), dim3(comb::NT), L,
                         po, part_lse, pl, (const uint16_t*)nullptr, o, lse_out, B, groups);
  return launch_kernel(combine_kernel<32, 64, 128, 128, true>, dim3(groups), dim3(comb::NT), L, po,
                       part_lse, pl, (const uint16_t*)nullptr, o, lse_out, B, groups);
}

hipError_t launch_combine(int shape, const void* part_o, const float* part_lse, const void* plan,
                          const int32_t* seq_lens, const void* W_UV, void* out, float* lse_out,
                          int B, int H, int max_pages, const Launch& L) {
  (void)seq_lens;
  (void)max_pages;
  const int groups = H * ((B + comb::SEQ - 1) / comb::SEQ);
  const uint16_t* po = (const uint16_t*)part_o;
  const Plan* pl = (const Plan*)plan;
  const uint16_t* w = (const uint16_t*)W_UV;
  uint16_t* o = (uint16_t*)out;
  if (shape == kShapeDeepSeek && groups >= comb::kWholeHeadGroups)
    return launch_kernel(combine_kernel<128, 512, 128, 128>, dim3(groups), dim3(comb::NT), L, po,
                         part_lse, pl, w, o, lse_out, B, groups);
  const int blocks = 16 * ((groups + 7) / 8);  // pairs of column halves, 8 ids apart
  if (shape == kShapeDeepSeek)
    return launch_kernel(combine_kernel<128, 512, 128, 64>, dim3(blocks), dim3(comb::NT), L, po,
                         part_lse, pl, w, o, lse_out, B, groups);
  return launch_kernel(combine_kernel<32, 64, 128, 64>, dim3(blocks), dim3(comb::NT), L, po,
                       part_lse, pl, w, o, lse_out, B, groups);
}

}  // namespace mla
