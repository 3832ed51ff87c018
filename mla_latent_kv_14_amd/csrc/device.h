// Device helpers shared by the gfx950 kernels: vector types, MFMA wrappers, LDS access,
// direct global->LDS loads, and the work plan that spreads the paged cache over work groups.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

#define MLA_LDS __attribute__((address_space(3)))

constexpr int kPage = 64;   // tokens per cache page
constexpr int kSub = 32;    // tokens per attention sub-tile (half a page)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------- MFMA (bf16 in, fp32 acc)
// 32x32x16: lane l holds A[l%32][8*(l/32)+j], B[8*(l/32)+j][l%32] (j < 8) and
//           D[8*(r/4) + 4*(l/32) + r%4][l%32] (r < 16).
__device__ __forceinline__ f32x16 mfma_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// 16x16x32: lane l holds A[l%16][8*(l/16)+j], B[8*(l/16)+j][l%16] (j < 8) and
//           D[4*(l/16) + r][l%16] (r < 4).
// Block-scaled 16x16x128 MFMA with FP8 (e4m3) A and B. A lane holds 32 bytes of row (A) or
// column (B) lane % 16, in the same order for both; the result is as for mfma_16x16x32 (lane:
// column lane % 16, rows 4(lane / 16) .. +4). sa and sb are E8M0 codes (operand times
// 2^(code - 127)), the same in the four lanes of a row or column.
__device__ __forceinline__ f32x4 mfma_scale_16x16x128_fp8(i32x8 a, i32x8 b, f32x4 c, int sa,
                                                          int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}
__device__ __forceinline__ f32x4 mfma_16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// 32x32x8: lane l holds A[l%32][4*(l/32)+j], B[4*(l/32)+j][l%32] (j < 4), D as 32x32x16.
__device__ __forceinline__ f32x16 mfma_32x32x8(i16x4 a, i16x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------- LDS access
__device__ __forceinline__ bf16x8 lds_read_b128(const MLA_LDS char* base, uint32_t byte_off) {
  return *reinterpret_cast<const MLA_LDS bf16x8*>(base + byte_off);
}
// Transposing LDS read: within each 16-lane group, lane i receives column i of a 4x16 block of
// 16-bit values whose row j is given by the 8-byte addresses of lanes 4j..4j+3 of the group.
__device__ __forceinline__ bf16x4 lds_read_tr16(const MLA_LDS char* base, uint32_t byte_off) {
  typedef MLA_LDS bf16x4 lds_bf16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(base + byte_off));
}
__device__ __forceinline__ bf16x8 cat4(bf16x4 lo, bf16x4 hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Direct global->LDS copy of 16 bytes per lane: lane l reads base + off_l (base uniform, in
// SGPRs) and its bytes land at lds + 16*l, so the whole wave writes one contiguous KiB (the LDS
// base goes in M0). Issued as inline assembly so that the compiler does not guard later LDS
// reads with a full vmcnt(0) drain: completion is tracked explicitly with wait_vmcnt<N>()
// before a block_sync().
__device__ __forceinline__ void load_lds_16(const void* base, uint32_t off, MLA_LDS void* lds) {
  const uint32_t m0 = (uint32_t)(uintptr_t)lds;
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "{m0}"(m0) : "memory");
}

// The same with 4 bytes per lane: LDS bytes [lds + 4*lane, +4) <- base + off.
__device__ __forceinline__ void load_lds_4(const void* base, uint32_t off, MLA_LDS void* lds) {
  const uint32_t m0 = (uint32_t)(uintptr_t)lds;
  asm volatile("global_load_lds_dword %0, %1" ::"v"(off), "s"(base), "{m0}"(m0) : "memory");
}

// 16-byte store at device scope (cache policy SC1): the line goes through this XCD's L2 to
// memory as it is stored instead of staying dirty there until the write-back that ends the
// kernel. Meant for a buffer that only the next kernel reads, from other XCDs (the split
// partials): the producer no longer ends on a burst of write-backs. base + byte_off is the
// address; the range check of the buffer descriptor is left wide open (2^31 - 1 bytes).
constexpr int kCacheSc1 = 16;  // the SC1 bit of a buffer instruction's cache-policy operand
__device__ __forceinline__ void store_16_device_scope(void* base, uint32_t byte_off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(
      v, __builtin_amdgcn_make_buffer_rsrc(base, 0, 0x7fffffff, 0x00020000), (int)byte_off, 0,
      kCacheSc1);
}
// The same for one 16-bit element (the coalescing of a wave's 64 lanes is unchanged).
__device__ __forceinline__ void store_2_device_scope(void* base, uint32_t byte_off, uint16_t v) {
  __builtin_amdgcn_raw_buffer_store_b16(
      v, __builtin_amdgcn_make_buffer_rsrc(base, 0, 0x7fffffff, 0x00020000), (int)byte_off, 0,
      kCacheSc1);
}

// Work-group barrier for LDS traffic only: waits for this wave's LDS operations, not for its
// outstanding global loads (the prefetched tiles stay in flight across the barrier).
__device__ __forceinline__ void block_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
// The same barrier with a distinct text per call site family: code paths of different waves
// that meet the barrier in different places (teams of a work group) keep their own copies, so
// the optimiser cannot merge them into one block (which would make both paths' registers live
// at once).
template <int TAG>
__device__ __forceinline__ void block_sync_tagged() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier ; team %0" ::"n"(TAG) : "memory");
}

// Read of a value that is the same for the whole wave from memory the kernel never writes:
// through the constant address space it becomes a scalar load (lgkmcnt, not vmcnt).
template <typename T>
__device__ __forceinline__ T ld_uniform(const T* p) {
  return *(const __attribute__((address_space(4))) T*)(p);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Marks a register as used here, so the compiler completes the load that produced it at this
// point (and knows it is complete afterwards) instead of at its later uses.
template <typename T>
__device__ __forceinline__ void settle(const T& v) {
  asm volatile("" ::"v"(v));
}

// Reductions over the lanes l, l^16, l^32, l^48 (the four 16-lane rows) with the gfx950 row
// swaps: v_permlane16_swap exchanges rows 1 and 3 of its first operand with rows 0 and 2 of its
// second, v_permlane32_swap the upper half of the first with the lower half of the second
// (checked on the device). Fed two copies of x, every lane ends with the pair {x[l], x[l^16]}
// (resp. {x[l], x[l^32]}), lower lane first, so the four lanes of a column get bit-identical
// results. VALU only, no LDS traffic. Written as inline assembly with both registers read and
// written (the compiler builtin returns the pair, but its second element is lost in code
// generation); the s_nop covers the wait after a VALU write of the operands.
__device__ __forceinline__ void swap_rows16(uint32_t& a, uint32_t& b) {
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void swap_halves32(uint32_t& a, uint32_t& b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ float rows4_max(float x) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  swap_rows16(a, b);
  uint32_t c = __builtin_bit_cast(uint32_t, fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b)));
  uint32_t d = c;
  swap_halves32(c, d);
  return fmaxf(__builtin_bit_cast(float, c), __builtin_bit_cast(float, d));
}
__device__ __forceinline__ float rows4_sum(float x) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  swap_rows16(a, b);
  uint32_t c = __builtin_bit_cast(uint32_t, __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b));
  uint32_t d = c;
  swap_halves32(c, d);
  return __builtin_bit_cast(float, c) + __builtin_bit_cast(float, d);
}

__device__ __forceinline__ float exp2f_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2f_fast(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ uint16_t bf16_bits(__bf16 x) { return __builtin_bit_cast(uint16_t, x); }
// Two floats rounded (RNE) to bf16 and packed, lo in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2 p = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, p);
}


// ---------------------------------------------------------------- work plan
// The cache of all sequences is viewed as one stream of tiles of TT tokens (32 for the DeepSeek
// widths, 64 for MHA2MLA), sequence after sequence, each sequence starting a new tile. Plan
// unit g of G owns tiles [g*per, min((g+1)*per, total)). The part of a sequence b that falls in
// unit g is a segment; its partial result goes to slot b + g, which is unique because the
// units that touch sequence b form a contiguous range that can share at most its first unit
// with sequence b-1. So a call needs at most G + B partial slots.
struct Plan {
  int32_t total;  // tiles over all sequences
  int32_t per;    // tiles per plan unit
  int32_t groups; // G
  int32_t pad;
  // followed by int32_t off[B]: first tile of sequence b,
  // then (at a 32-byte boundary) UnitStart start[G]
};
// Where plan unit g starts, written for every unit, so that a work group finds its tile count,
// its first tile, that tile's sequence and page with one scalar load and no other dependency.
struct UnitStart {
  int32_t b;     // sequence holding the unit's first tile
  int32_t j;     // that tile's index inside the sequence
  int32_t nj;    // tiles of sequence b
  int32_t S;     // clamped length of sequence b
  int32_t page;  // page-table entry of the page holding tile j (as stored; clamped at use)
  int32_t n;     // tiles the unit owns; 0 for an idle unit (whose other fields are 0)
  int32_t pad[2];
};
__device__ __forceinline__ const int32_t* plan_off(const Plan* p) {
  return reinterpret_cast<const int32_t*>(p + 1);
}
__device__ __forceinline__ int32_t* plan_off(Plan* p) { return reinterpret_cast<int32_t*>(p + 1); }
__host__ __device__ constexpr size_t plan_units_offset(int B) {
  return (sizeof(Plan) + 4 * (size_t)B + 31) & ~(size_t)31;
}
__host__ __device__ constexpr size_t plan_bytes(int B, int G) {
  return plan_units_offset(B) + sizeof(UnitStart) * (size_t)G;
}
__device__ __forceinline__ const UnitStart* plan_units(const Plan* p, int B) {
  return reinterpret_cast<const UnitStart*>(reinterpret_cast<const char*>(p) + plan_units_offset(B));
}
__device__ __forceinline__ UnitStart* plan_units(Plan* p, int B) {
  return reinterpret_cast<UnitStart*>(reinterpret_cast<char*>(p) + plan_units_offset(B));
}
// The unit record through the scalar path (written by an earlier kernel, read-only here), as
// one 32-byte load: no field waits for a second round trip, whatever branches on which field.
__device__ __forceinline__ UnitStart load_unit(const Plan* p, int B, int g) {
  const i32x8 w = ld_uniform(reinterpret_cast<const i32x8*>(plan_units(p, B) + g));
  UnitStart u;
  u.b = w[0];
  u.j = w[1];
  u.nj = w[2];
  u.S = w[3];
  u.page = w[4];
  u.n = w[5];
  return u;
}

// Effective S_b: clamped to what the page table row can address.
__device__ __forceinline__ int clamp_len(int s, int max_pages) {
  s = s < 0 ? 0 : s;
  int cap = max_pages * kPage;
  return s > cap ? cap : s;
}

// Several query tokens per sequence (q_len of them: the sequence's newest tokens, already in
// the cache) are decoded as virtual sequences v = b * q_len + i, i < q_len. Virtual sequence v
// reads row b of the page table and sees the first S_b - (q_len - 1 - i) tokens: each query
// token attends to itself and to every earlier token. With q_len = 1, v = b.
__device__ __forceinline__ int virt_row(int v, int q_len) { return q_len == 1 ? v : v / q_len; }
// Length of virtual sequence v, given the clamped length of its page-table row.
__device__ __forceinline__ int virt_len(int row_len, int v, int q_len) {
  if (q_len == 1) return row_len;
  const int s = row_len - (q_len - 1 - (v - (v / q_len) * q_len));
  return s > 0 ? s : 0;
}

}  // namespace mla
