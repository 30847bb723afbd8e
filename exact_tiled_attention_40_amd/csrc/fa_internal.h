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
};

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
