// Internal interface between the C-ABI front end (fa_api.cpp) and the
// kernel launchers.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

struct AttnShape {
  int B, H, N, d;
  int64_t ld;              // elements between consecutive tokens of q, k, v, dq, dk, dv
  const int32_t* cu;       // device prefix sums (varlen) or nullptr
  bool causal;
  bool bf16;
  float scale;
  bool dropout;
  uint32_t drop_thresh;    // floor(p * 2^16)
  float drop_rescale;      // 1 / (1 - p)
  uint64_t seed;
  const uint8_t* bmask;    // block mask [B, H, nb, nb] (device) or nullptr: dense
  int nb;                  // mask blocks per side, ceil(N / 128)
  // Dropout keep bits (device; dense and varlen only) or nullptr: the
  // forward stores the decisions it draws, the backward reads them instead
  // of hashing.  Word (((b*H + h) * nkt + t) * 2 + w) * Np + i holds, in bit
  // k, the decision of query i against key 64t + 32w + k (local indices,
  // nkt = ceil(N / 64), Np = N rounded up to a multiple of 4, so that every
  // run of four rows the kernels move is 16-byte aligned).
  uint32_t* keep_bits;
};

// Row stride (words) of the keep-bit planes of sequences of at most N tokens.
inline int keep_bits_rows(int N) { return (N + 3) & ~3; }

// Number of 32-bit words of the keep-bit buffer of B sequences of at most N
// tokens with H heads (0 if it overflows 64 bits).
inline uint64_t keep_bits_words(int B, int N, int H) {
  const uint64_t nkt = ((uint64_t)N + 63) / 64;
  const uint64_t heads = (uint64_t)B * (uint64_t)H;
  if (heads == 0 || nkt == 0 || N < 1) return 0;
  const uint64_t per_head = nkt * 2 * (uint64_t)keep_bits_rows(N);
  if (per_head > UINT64_MAX / 8 / heads) return 0;
  return per_head * heads;
}

// First token and length of sequence b of a batch of B sequences whose
// longest is N.  Fixed length: b*N and N.  Varlen: from the prefix sums cu
// (cu[b] .. cu[b+1] - 1 are the sequence's tokens, cu[B] tokens in all),
// clamped so that every token index the kernels form lies in
// [0, min(cu[B], B*N)): a sequence longer than N is cut to its first N
// tokens (the grid and the tile lists are sized for N), and prefix sums that
// are not monotone or exceed B*N (the rows of the backward workspace) give
// empty or shortened sequences instead of accesses out of bounds.
__host__ __device__ inline void seq_bounds(const int32_t* cu, int b, int B, int N, int& start, int& L) {
  if (!cu) {
    start = b * N;
    L = N;
    return;
  }
  const int cap = B * N;  // fits in int32: checked on the host
  int total = cu[B];
  total = total < 0 ? 0 : (total > cap ? cap : total);
  int s = cu[b];
  s = s < 0 ? 0 : (s > total ? total : s);
  int e = cu[b + 1];
  const int e_max = (total - s < N) ? total : s + N;
  e = e < s ? s : (e > e_max ? e_max : e);
  start = s;
  L = e - s;
}

hipError_t launch_forward(const AttnShape& s, const void* q, const void* k, const void* v, void* o,
                          float* lse, hipStream_t stream);

hipError_t launch_backward(const AttnShape& s, const void* q, const void* k, const void* v,
                           const void* o, const float* lse, const void* dout, void* dq, void* dk,
                           void* dv, float* delta, float* lse2, int stages,
                           hipStream_t stream);

// Stage bits of launch_backward: the dQ kernel (which also writes D) and the
// dK/dV kernel (which reads D).
constexpr int kBwdDq = 1, kBwdKV = 2, kBwdAll = 3;

// KV-cache decode step: nq new queries per sequence against its cache.
struct DecodeShape {
  int B, H, nq, nk, d;  // nk = cache capacity (tokens) per sequence
  bool causal;
  bool bf16;
  float scale;
};

// Number of 1024-key chunks (split workgroups) of a cache of nk tokens.
int decode_splits(int nk);

// workspace: fp32, B*H*decode_splits(nk)*nq*(d + 2) floats.
// A paged cache: pools of num_pages pages of page_size tokens (a power of
// two) and a device table [B, max_pages] of page numbers; nk of the shape is
// max_pages * page_size.
struct DecodePages {
  const int32_t* table;
  int page_size, max_pages, num_pages;
};

hipError_t launch_decode(const DecodeShape& s, const void* q, const void* k, const void* v, const int32_t* lk,
                         void* o, float* lse, float* workspace, hipStream_t stream,
                         const DecodePages* pages = nullptr);

hipError_t launch_dropout_mask(uint8_t* keep, int b, int h, int N, uint32_t thresh, uint64_t seed,
                               hipStream_t stream);

}  // namespace fa
