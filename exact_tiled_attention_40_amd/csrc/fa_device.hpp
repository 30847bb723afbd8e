// Device-side building blocks shared by the gfx950 attention kernels:
// vector types, MFMA wrappers, LDS transpose reads, 16-bit packing, wave-half
// reductions and the Philox-4x32-10 dropout hash.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa.h"

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// D += A * B on a 32x32 tile with a K slice of 16 (bf16 or fp16 inputs,
// fp32 accumulation).  Lane l holds A row l%32, B column l%32, and K
// elements 8*(l/32) .. 8*(l/32)+7 of each; the accumulator register r of
// lane l is element (row 8*(r/4) + 4*(l/32) + r%4, column l%32).
template <bool BF16>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (BF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Two fp32 values -> two 16-bit floats (round to nearest even) in one word.
template <bool BF16>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  if constexpr (BF16) {
    bf16x2 v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
  } else {
    f16x2 v = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, v);
  }
}

template <bool BF16>
__device__ __forceinline__ float to_f32(uint16_t x) {
  if constexpr (BF16) return __builtin_bit_cast(float, (uint32_t)x << 16);
  else return (float)__builtin_bit_cast(_Float16, x);
}

// Buffer resource over `bytes` bytes from `base`: raw buffer loads at
// offsets at or past `bytes` return zeros (the hardware range check), which is
// how ragged tails are zero-filled without branches.
// base and bytes must be wave-uniform; they are read from the first lane so
// that the descriptor is known to live in scalar registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t p = (uint64_t)(uintptr_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
  void* ub = (void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(ub, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t voffset) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voffset, 0, 0));
}

// 16-byte buffer load of every lane straight into LDS: lane l's 16 bytes land
// at byte address lds_base + 16*l (lds_base must be wave-uniform).  Issued
// from inline assembly so that the compiler does not wait for it before
// unrelated LDS reads (it cannot tell the double buffers apart); callers wait
// with wait_vmem() before a barrier.  M0 (the LDS base register) is declared
// clobbered, so the compiler sets it again wherever it needs it itself.
__device__ __forceinline__ void buffer_load_lds16_addr(__amdgpu_buffer_rsrc_t r, uint32_t lds_base, uint32_t voffset) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds"
      :
      : "s"(lds_base), "v"(voffset), "s"(r)
      : "memory", "m0");
}

// 4-byte buffer load of every lane straight into LDS: lane l's 4 bytes land
// at lds_base + 4*l.  Same conventions as buffer_load_lds16_addr.
__device__ __forceinline__ void buffer_load_lds4(__amdgpu_buffer_rsrc_t r, const void* lds_base, uint32_t voffset) {
  const uint32_t base = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)lds_base;
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %1, %2, 0 offen lds"
      :
      : "s"(base), "v"(voffset), "s"(r)
      : "memory", "m0");
}

// LDS address (bytes) of a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

__device__ __forceinline__ u32x4 lds_read16_at(uint32_t addr) {
  return *(const __attribute__((address_space(3))) u32x4*)(uintptr_t)addr;
}

// LDS transpose read (ds_read_b64_tr_b16) at a byte address.  Within each group of 16 lanes,
// source lane s supplies the address of four consecutive 16-bit elements;
// destination lane l receives element l%4 of source lanes 4e + l/4 (e = 0..3).
// Pointed at a row-major [k][n] tile with lane s addressing row k0 + s/4,
// columns n0 + 4*(s%4) .. +3, lane l gets column n0 + l%16, rows k0 .. k0+3.
__device__ __forceinline__ u32x2 lds_read_tr_at(uint32_t addr) {
  s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(uintptr_t)addr);
  return __builtin_bit_cast(u32x2, v);
}

// buffer_load_lds4 with the LDS destination given as a byte address.
__device__ __forceinline__ void buffer_load_lds4_addr(__amdgpu_buffer_rsrc_t r, uint32_t lds_base, uint32_t voffset) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %1, %2, 0 offen lds"
      :
      : "s"(lds_base), "v"(voffset), "s"(r)
      : "memory", "m0");
}

// MI355X: 8 XCDs, each with its own L2; the hardware deals a launch's
// workgroups to them in turn.
constexpr int kXcds = 8;

// Workgroup id -> (head bh = b*H + h, rank among the head's per_head
// workgroups).  With heads fastest, workgroup i lands on XCD i % 8, so all
// workgroups of one head share an XCD (and its L2) whenever B*H is a
// multiple of 8.  When B*H is a multiple of 8*G, XCD x moreover takes its
// heads (x, x + 8, ...) G at a time, ranks in order with the G heads
// alternating, so that its L2 serves the tiles of G heads at a time instead
// of all of its heads at once.
template <int G>
__device__ __forceinline__ void xcd_head_order(int id, int BH, int per_head, int& bh, int& rank) {
  if (BH % (kXcds * G) == 0) {
    const int m = id / kXcds;
    const int g = m / (G * per_head), r = m % (G * per_head);
    bh = id % kXcds + kXcds * (g * G + r % G);
    rank = r / G;
  } else {
    bh = id % BH;
    rank = id / BH;
  }
}

// ------------------------------------------------------- block-sparse lists
// Block masks have square blocks of kMaskBlock rows (queries) by kMaskBlock
// columns (keys); the kernels' 64-row tiles are halves of mask blocks.
constexpr int kMaskBlock = 128;
constexpr int kMaxSparseTiles = 1024;  // 64-row tiles per sequence (N <= 65536)
static_assert(kMaskBlock == FA_MASK_BLOCK && kMaxSparseTiles * 64 == FA_MASK_MAX_N,
              "block-mask geometry must match the C ABI");

// Compacted list of the tiles one workgroup visits under a block mask, built
// by a single wave.  Tile t (0 <= t < ntiles) reads mask byte
// ((t0 + t) / 2) * stride of row m0 and, if m1 is not null, of row m1; it is
// listed when either byte is nonzero, with flag bit 0 / bit 1 set for a
// nonzero byte of m0 / m1.  Returns the number of listed tiles (uniform).
__device__ __forceinline__ int build_tile_list(const uint8_t* m0, const uint8_t* m1, int t0, int64_t stride,
                                               int ntiles, uint16_t* list, uint8_t* flags, int lane) {
  int n = 0;
  for (int base = 0; base < ntiles; base += 64) {
    const int t = base + lane;
    int f = 0;
    if (t < ntiles) {
      const int64_t off = (int64_t)((t0 + t) >> 1) * stride;
      f = (m0[off] != 0 ? 1 : 0) | (m1 != nullptr && m1[off] != 0 ? 2 : 0);
    }
    const uint64_t bal = __builtin_amdgcn_ballot_w64(f != 0);
    const int pos = n + __builtin_popcountll(bal & ((1ull << lane) - 1ull));
    if (f != 0) {
      list[pos] = (uint16_t)t;
      flags[pos] = (uint8_t)f;
    }
    n += __builtin_popcountll(bal);
  }
  return n;
}

// A tile of ROWS rows (a multiple of 32) of D 16-bit elements in LDS, laid
// out for the two ways the MFMA loops read it:
//   - operand read: lane l of a wave takes the 16-byte chunk 2s + l/32 of row
//     32g + l%32 (a 32x32x16 A or B operand with rows on lanes);
//   - transpose read (ds_read_b64_tr_b16): 16 lanes take four consecutive
//     elements each of 4 rows, so that every lane receives one column of a
//     4-row slice (an operand with rows on the K dimension).
// The tile is split into 1 KB blocks, block (g, s) holding chunks 2s, 2s + 1
// of rows 32g .. 32g + 31; inside a block, logical slot x = row%32 + 32*(chunk
// % 2) sits at physical 16-byte slot x ^ 4*(x/32) ^ 8*(s%2).  An operand read
// is then 64 consecutive slots (permuted inside each 16-slot group), and a
// transpose read hits 32 different 8-byte bank pairs per half-wave, so
// neither conflicts with 64 four-byte banks; and every read of a loop is one
// per-lane base register plus an immediate offset.  Blocks are filled whole
// by 1 KB direct-to-LDS loads (lane l writes physical slot l).
template <int D, int ROWS>
struct MTile {
  static constexpr int kSPR = D / 16;                  // blocks per 32-row group
  static constexpr int kBlocks = ROWS / 32 * kSPR;     // = number of 1 KB loads
  static constexpr int kElems = kBlocks * 512;         // 16-bit elements
  static constexpr int kBytes = kBlocks * 1024;

  // Load block u: lane l fetches the chunk that belongs at physical slot l.
  // row_bytes apart rows; rows the buffer range does not cover read as 0.
  __device__ static __forceinline__ void load(__amdgpu_buffer_rsrc_t rsrc, uint32_t tile_addr, uint32_t row_bytes,
                                              int u, int lane) {
    const int s = u % kSPR;
    const int g = u / kSPR;
    const int x = lane ^ ((lane >> 5) << 2) ^ ((s & 1) << 3);
    const uint32_t off = (uint32_t)(32 * g + (x & 31)) * row_bytes + 16 * (2 * s + (x >> 5));
    buffer_load_lds16_addr(rsrc, tile_addr + 1024 * u, off);
  }
  // Operand read of block (g, s) = tile + opnd_off(g, s) + opnd_base(lane, s % 2).
  __device__ static __forceinline__ uint32_t opnd_base(int lane, int sodd) {
    return 16 * (lane ^ ((lane >> 5) << 2) ^ (sodd << 3));
  }
  static constexpr uint32_t opnd_off(int g, int s) { return 1024 * (g * kSPR + s); }
  // Transpose read of rows 16m + 8hi + 4*(lane/32) + 0..3, columns 32dt + lane%32:
  // tile + tr_off(m, dt) + tr_base(lane, hi).
  __device__ static __forceinline__ uint32_t tr_base(int lane, int hi) {
    const int g = (lane >> 4) & 1, h2 = lane >> 5, sl = lane & 15;
    const int e = sl >> 2, f = (sl >> 1) & 1, half = sl & 1;
    const int x = (8 * hi + 4 * h2 + e + 32 * f) ^ (4 * f) ^ (8 * g);
    return 1024 * g + 16 * x + 8 * half;
  }
  static constexpr uint32_t tr_off(int m, int dt) { return 1024 * ((m >> 1) * kSPR + 2 * dt) + 256 * (m & 1); }
};

// Wait until this wave's outstanding vector-memory operations (including
// direct-to-LDS loads) have completed.
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Wait until at most N of this wave's vector-memory operations are
// outstanding (loads complete in issue order, so the older ones are done).
template <int N>
__device__ __forceinline__ void wait_vmem_n() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier without the LDS fence of __syncthreads(), for loops whose
// only LDS writes are direct-to-LDS loads (completed by wait_vmem() before
// the barrier): LDS reads issued before it may stay in flight.  The memory
// clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void barrier_keep_lds_reads() { asm volatile("s_barrier" ::: "memory"); }

// v_permlane32_swap: lanes 32-63 of a trade places with lanes 0-31 of b.
// Written as inline assembly because the compiler's builtin for it returns
// the first operand for both results.  The s_nop covers the VALU-write ->
// permlane-read hazard.
__device__ __forceinline__ void permlane32_swap(uint32_t& a, uint32_t& b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}

// Reductions over lanes l and l ^ 32, result in every lane: swapping x with
// a copy of itself leaves the low half's values in a and the high half's in b.
__device__ __forceinline__ float halves_max(float x) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  permlane32_swap(a, b);
  return fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}

__device__ __forceinline__ float halves_sum(float x) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  permlane32_swap(a, b);
  return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
}

// Value of lane 4*(l/4) + Pk in lane l (k = l mod 4): a DPP quad
// permutation (every lane of the quad must be active).
template <int P0, int P1, int P2, int P3>
__device__ __forceinline__ uint32_t quad_perm(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, P0 | (P1 << 2) | (P2 << 4) | (P3 << 6), 0xf, 0xf, false);
}

// Philox-4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of the
// multiply-xor round function with a Weyl-sequence key schedule.
struct Philox4 {
  uint32_t x, y, z, w;
};

// Round r (0-based) of Philox-4x32-10 on the counter state c with key
// (k0, k1): the round key is the key advanced r times by the Weyl constants.
// Each 32x32 -> 64-bit product is one v_mad_u64_u32 (high and low halves),
// each three-way xor one v_bitop3_b32.
__device__ __forceinline__ void philox_round(uint32_t (&c)[4], uint32_t k0, uint32_t k1, int r) {
  const uint32_t rk0 = k0 + (uint32_t)r * 0x9E3779B9u, rk1 = k1 + (uint32_t)r * 0xBB67AE85u;
  const uint64_t p0 = (uint64_t)0xD2511F53u * c[0];
  const uint64_t p1 = (uint64_t)0xCD9E8D57u * c[2];
  const uint32_t n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c[1], rk0, 0x96);
  const uint32_t n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c[3], rk1, 0x96);
  c[0] = n0;
  c[1] = (uint32_t)p1;
  c[2] = n2;
  c[3] = (uint32_t)p0;
}

__device__ __forceinline__ Philox4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                                 uint32_t k0, uint32_t k1) {
  uint32_t c[4] = {c0, c1, c2, c3};
#pragma unroll
  for (int r = 0; r < 10; ++r) philox_round(c, k0, k1, r);
  return {c[0], c[1], c[2], c[3]};
}

// Dropout keep decision of one element from its 16-bit Philox value: the
// low (hi = 0) or high (hi = 1) half of word w, kept iff >= thresh.
__device__ __forceinline__ bool keep16(uint32_t w, int hi, uint32_t thresh) {
  return (hi ? w >> 16 : w & 0xFFFFu) >= thresh;
}

// Keep words of one query against two aligned 8-key groups, for layouts in
// which lane half h2 holds keys 4*h2 .. 4*h2+3 of every group (lanes l and
// l^32 own the same query qi).  The block with counter (qi, group, h, b)
// holds the 16-bit values of the group's eight keys (value v: half v%2 of
// word v/2), so a lane half needs two of its four words.  The two lanes of
// a query split the work: lane half h2 hashes group j8/8 + h2 (j8: first key
// of the pair), and one permlane32 swap per word pair trades the halves.  On
// return kw[u][0..1] are this lane's words of group j8/8 + u.
__device__ __forceinline__ void keep_words_pair(int qi, int j8, int h2, int h, int b, uint32_t seed_lo,
                                                uint32_t seed_hi, uint32_t (&kw)[2][2]) {
  const Philox4 r = philox4x32_10((uint32_t)qi, (uint32_t)(j8 >> 3) + (uint32_t)h2, (uint32_t)h, (uint32_t)b,
                                  seed_lo, seed_hi);
  // lanes 0-31 keep x, y of their group (j8/8) and send z, w; lanes 32-63
  // keep z, w of theirs (j8/8 + 1) and send x, y
  uint32_t a0 = r.x, b0 = r.z, a1 = r.y, b1 = r.w;
  permlane32_swap(a0, b0);
  permlane32_swap(a1, b1);
  kw[0][0] = a0;
  kw[0][1] = a1;
  kw[1][0] = b0;
  kw[1][1] = b1;
}

}  // namespace fa
