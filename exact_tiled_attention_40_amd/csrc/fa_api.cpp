// C-ABI front end of libfa: argument validation (host only, before any HIP
// call), dtype/shape dispatch and workspace carving.  Every entry point
// returns an fa_status code; none allocates, synchronizes or aborts.
#include "../../include/fa.h"

#include <cmath>
#include <cstdint>
#include <mutex>

#include "fa_internal.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shared checks of fa_forward / fa_backward; fills the launch description.
int check_common(int B, int H, int N, int d, float scale, float dropout_p, int dtype, int64_t ld_qkv,
                 const int32_t* cu_seqlens, int causal, uint64_t seed, fa::AttnShape* s) {
  if (dtype != FA_DTYPE_F16 && dtype != FA_DTYPE_BF16) return FA_ERR_UNSUPPORTED;
  if (d != 32 && d != 64 && d != 96 && d != 128 && d != 160 && d != 192 && d != 256) return FA_ERR_UNSUPPORTED;
  if (B < 1 || H < 1 || N < 1) return FA_ERR_BAD_SHAPE;
  // all token offsets must fit in 32-bit signed ints (B*N tokens) and byte
  // offsets in 64 bits
  if ((int64_t)B * N > INT32_MAX) return FA_ERR_BAD_SHAPE;
  if (!std::isfinite(scale) || !(scale > 0.f)) return FA_ERR_BAD_ARGUMENT;
  if (!(dropout_p >= 0.f) || !(dropout_p < 1.f)) return FA_ERR_BAD_ARGUMENT;
  const int64_t hd = (int64_t)H * d;
  const int64_t ld = ld_qkv == 0 ? hd : ld_qkv;
  if (ld < hd || (ld % 8) != 0) return FA_ERR_ALIGNMENT;
  // the kernels address a 64-token tile through a 32-bit buffer range
  if (ld > FA_MAX_TOKEN_STRIDE) return FA_ERR_UNSUPPORTED;
  if (cu_seqlens && (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u)) return FA_ERR_ALIGNMENT;
  s->B = B;
  s->H = H;
  s->N = N;
  s->d = d;
  s->ld = ld;
  s->cu = cu_seqlens;
  s->causal = causal != 0;
  s->bf16 = dtype == FA_DTYPE_BF16;
  s->scale = scale;
  s->dropout = dropout_p > 0.f;
  const double t = std::floor((double)dropout_p * 65536.0);
  s->drop_thresh = s->dropout ? (uint32_t)t : 0u;
  s->drop_rescale = s->dropout ? 1.0f / (1.0f - dropout_p) : 1.0f;
  s->seed = seed;
  s->bmask = nullptr;
  s->nb = 0;
  s->keep_bits = nullptr;
  return FA_OK;
}

// Block-sparse additions to a checked launch description.
int check_block_mask(const uint8_t* block_mask, int N, fa::AttnShape* s) {
  if (!block_mask) return FA_ERR_NULL_POINTER;
  if (N > FA_MASK_MAX_N) return FA_ERR_UNSUPPORTED;
  s->bmask = block_mask;
  s->nb = (N + FA_MASK_BLOCK - 1) / FA_MASK_BLOCK;
  return FA_OK;
}

}  // namespace

extern "C" {

// Keep-bit additions to a checked launch description (the bits matter only
// with dropout).
static int check_keep_bits(const void* bits, size_t bytes, fa::AttnShape* s) {
  if (!s->dropout) return FA_OK;
  if (!bits) return FA_ERR_NULL_POINTER;
  if (s->N > FA_MASK_MAX_N) return FA_ERR_UNSUPPORTED;
  const size_t need = fa_dropout_bits_size(s->B, s->N, s->H);
  if (need == 0 || bytes < need) return FA_ERR_WORKSPACE;
  if (!aligned16(bits)) return FA_ERR_ALIGNMENT;
  s->keep_bits = const_cast<uint32_t*>(static_cast<const uint32_t*>(bits));
  return FA_OK;
}

static int forward_impl(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
                        int d, float scale, int causal, const int32_t* cu_seqlens, float dropout_p, uint64_t seed,
                        void* stream, int dtype, int64_t ld_qkv, const uint8_t* block_mask, bool sparse,
                        uint32_t* keep_bits = nullptr, size_t keep_bits_bytes = 0, bool keep = false) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL_POINTER;
  fa::AttnShape s;
  int rc = check_common(B, H, N, d, scale, dropout_p, dtype, ld_qkv, cu_seqlens, causal, seed, &s);
  if (rc != FA_OK) return rc;
  if (sparse && (rc = check_block_mask(block_mask, N, &s)) != FA_OK) return rc;
  if (keep && (rc = check_keep_bits(keep_bits, keep_bits_bytes, &s)) != FA_OK) return rc;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return FA_ERR_ALIGNMENT;
  const hipError_t e = fa::launch_forward(s, q, k, v, o, lse, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_forward(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
               float scale, int causal, const int32_t* cu_seqlens, float dropout_p, uint64_t seed, void* stream,
               int dtype, int64_t ld_qkv) {
  return forward_impl(q, k, v, o, lse, B, H, N, d, scale, causal, cu_seqlens, dropout_p, seed, stream, dtype,
                      ld_qkv, nullptr, false);
}

int fa_forward_block_sparse(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                            int N, int d, float scale, int causal, const int32_t* cu_seqlens, float dropout_p,
                            uint64_t seed, void* stream, int dtype, int64_t ld_qkv, const uint8_t* block_mask) {
  return forward_impl(q, k, v, o, lse, B, H, N, d, scale, causal, cu_seqlens, dropout_p, seed, stream, dtype,
                      ld_qkv, block_mask, true);
}

int fa_forward_keep(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
                    float scale, int causal, const int32_t* cu_seqlens, float dropout_p, uint64_t seed,
                    void* stream, int dtype, int64_t ld_qkv, uint32_t* keep_bits, size_t keep_bits_bytes) {
  return forward_impl(q, k, v, o, lse, B, H, N, d, scale, causal, cu_seqlens, dropout_p, seed, stream, dtype,
                      ld_qkv, nullptr, false, keep_bits, keep_bits_bytes, true);
}

size_t fa_dropout_bits_size(int B, int N, int H) {
  if (B < 1 || N < 1 || H < 1 || N > FA_MASK_MAX_N) return 0;
  const uint64_t words = fa::keep_bits_words(B, N, H);
  if (words == 0 || words > SIZE_MAX / 4) return 0;
  return (size_t)(words * 4);
}

size_t fa_backward_workspace_size(int B, int N, int H, int d) {
  if (B < 1 || N < 1 || H < 1 || d < 1) return 0;
  const uint64_t rows = (uint64_t)B * (uint64_t)N * (uint64_t)H;
  if (rows > ((UINT64_MAX - 255) / 4) / 2) return 0;
  // D = rowsum(dO * O) and LSE * log2(e): fp32 [B*N, H] each, each rounded up
  // to 256 bytes
  return (size_t)(2 * ((rows * 4 + 255) & ~(uint64_t)255));
}

// Checks of the backward's tensors and sizes (everything but the workspace).
static int check_backward(const void* q, const void* k, const void* v, const void* o, const float* lse,
                          const void* dout, void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale,
                          int causal, const int32_t* cu_seqlens, float dropout_p, uint64_t seed, int dtype,
                          int64_t ld_qkv, const uint8_t* block_mask, bool sparse, fa::AttnShape* s) {
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return FA_ERR_NULL_POINTER;
  int rc = check_common(B, H, N, d, scale, dropout_p, dtype, ld_qkv, cu_seqlens, causal, seed, s);
  if (rc != FA_OK) return rc;
  if (sparse && (rc = check_block_mask(block_mask, N, s)) != FA_OK) return rc;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) ||
      !aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return FA_ERR_ALIGNMENT;
  return FA_OK;
}

// Enqueues the backward with its two row arrays carved from `workspace`
// (D first, then lse * log2(e) at the next 256-byte boundary).
static int launch_backward_ws(const fa::AttnShape& s, int stages, const void* q, const void* k, const void* v,
                              const void* o, const float* lse, const void* dout, void* dq, void* dk, void* dv,
                              void* workspace, void* stream) {
  float* delta = static_cast<float*>(workspace);
  const uint64_t rows = (uint64_t)s.B * (uint64_t)s.N * (uint64_t)s.H;
  float* lse2 = delta + ((rows * 4 + 255) & ~(uint64_t)255) / 4;
  const hipError_t e = fa::launch_backward(s, q, k, v, o, lse, dout, dq, dk, dv, delta, lse2, stages,
                                           static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

static int backward_impl(int stages, const void* q, const void* k, const void* v, const void* o, const float* lse,
                         const void* dout, void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale,
                         int causal, const int32_t* cu_seqlens, float dropout_p, uint64_t seed, void* stream,
                         int dtype, int64_t ld_qkv, void* workspace, size_t workspace_bytes,
                         const uint8_t* block_mask, bool sparse, const uint32_t* keep_bits = nullptr,
                         size_t keep_bits_bytes = 0, bool keep = false) {
  fa::AttnShape s;
  int rc = check_backward(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, d, scale, causal, cu_seqlens, dropout_p,
                          seed, dtype, ld_qkv, block_mask, sparse, &s);
  if (rc != FA_OK) return rc;
  if (keep && (rc = check_keep_bits(keep_bits, keep_bits_bytes, &s)) != FA_OK) return rc;
  const size_t need = fa_backward_workspace_size(B, N, H, d);
  if (!workspace || need == 0 || workspace_bytes < need) return FA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return FA_ERR_ALIGNMENT;
  return launch_backward_ws(s, stages, q, k, v, o, lse, dout, dq, dk, dv, workspace, stream);
}

int fa_backward(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale, int causal,
                const int32_t* cu_seqlens, float dropout_p, uint64_t seed, void* stream, int dtype, int64_t ld_qkv,
                void* workspace, size_t workspace_bytes) {
  return backward_impl(fa::kBwdAll, q, k, v, o, lse, dout, dq, dk, dv, B, H, N, d, scale, causal, cu_seqlens,
                       dropout_p, seed, stream, dtype, ld_qkv, workspace, workspace_bytes, nullptr, false);
}

int fa_backward_keep(const void* q, const void* k, const void* v, const void* o, const float* lse,
                     const void* dout, void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale,
                     int causal, const int32_t* cu_seqlens, float dropout_p, uint64_t seed, void* stream, int dtype,
                     int64_t ld_qkv, void* workspace, size_t workspace_bytes, const uint32_t* keep_bits,
                     size_t keep_bits_bytes) {
  return backward_impl(fa::kBwdAll, q, k, v, o, lse, dout, dq, dk, dv, B, H, N, d, scale, causal, cu_seqlens,
                       dropout_p, seed, stream, dtype, ld_qkv, workspace, workspace_bytes, nullptr, false, keep_bits,
                       keep_bits_bytes, true);
}

int fa_backward_keep_stage(int stage, const void* q, const void* k, const void* v, const void* o, const float* lse,
                           const void* dout, void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale,
                           int causal, const int32_t* cu_seqlens, float dropout_p, uint64_t seed, void* stream,
                           int dtype, int64_t ld_qkv, void* workspace, size_t workspace_bytes,
                           const uint32_t* keep_bits, size_t keep_bits_bytes) {
  if (stage < 0 || stage > 1) return FA_ERR_BAD_ARGUMENT;
  return backward_impl(1 << stage, q, k, v, o, lse, dout, dq, dk, dv, B, H, N, d, scale, causal, cu_seqlens,
                       dropout_p, seed, stream, dtype, ld_qkv, workspace, workspace_bytes, nullptr, false, keep_bits,
                       keep_bits_bytes, true);
}

int fa_backward_block_sparse(const void* q, const void* k, const void* v, const void* o, const float* lse,
                             const void* dout, void* dq, void* dk, void* dv, int B, int H, int N, int d,
                             float scale, int causal, const int32_t* cu_seqlens, float dropout_p, uint64_t seed,
                             void* stream, int dtype, int64_t ld_qkv, void* workspace, size_t workspace_bytes,
                             const uint8_t* block_mask) {
  return backward_impl(fa::kBwdAll, q, k, v, o, lse, dout, dq, dk, dv, B, H, N, d, scale, causal, cu_seqlens,
                       dropout_p, seed, stream, dtype, ld_qkv, workspace, workspace_bytes, block_mask, true);
}

int fa_backward_stage(int stage, const void* q, const void* k, const void* v, const void* o, const float* lse,
                      const void* dout, void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale,
                      int causal, const int32_t* cu_seqlens, float dropout_p, uint64_t seed, void* stream,
                      int dtype, int64_t ld_qkv, void* workspace, size_t workspace_bytes) {
  if (stage < 0 || stage > 1) return FA_ERR_BAD_ARGUMENT;
  return backward_impl(1 << stage, q, k, v, o, lse, dout, dq, dk, dv, B, H, N, d, scale, causal, cu_seqlens,
                       dropout_p, seed, stream, dtype, ld_qkv, workspace, workspace_bytes, nullptr, false);
}

int fa_backward_block_sparse_stage(int stage, const void* q, const void* k, const void* v, const void* o,
                                   const float* lse, const void* dout, void* dq, void* dk, void* dv, int B, int H,
                                   int N, int d, float scale, int causal, const int32_t* cu_seqlens,
                                   float dropout_p, uint64_t seed, void* stream, int dtype, int64_t ld_qkv,
                                   void* workspace, size_t workspace_bytes, const uint8_t* block_mask) {
  if (stage < 0 || stage > 1) return FA_ERR_BAD_ARGUMENT;
  return backward_impl(1 << stage, q, k, v, o, lse, dout, dq, dk, dv, B, H, N, d, scale, causal, cu_seqlens,
                       dropout_p, seed, stream, dtype, ld_qkv, workspace, workspace_bytes, block_mask, true);
}

// ---------------------------------------------------- no-allocation backward
// The backward's workspace (D and lse * log2(e), fp32 [B*N, H] each) for
// callers that cannot allocate: a fixed array in device memory, one copy per
// GPU, held from the first call on that GPU until the process ends.  Host
// code only ever uses the address hipGetSymbolAddress returns for the GPU
// (the array's name is a host-side stand-in, not a device address).
static __device__ __align__(256) unsigned char scratch[FA_NOALLOC_SCRATCH_BYTES];
static_assert(FA_NOALLOC_SCRATCH_BYTES == 2 * (size_t)FA_NOALLOC_MAX_ROWS * 4,
              "two fp32 arrays of FA_NOALLOC_MAX_ROWS rows, each a multiple of 256 bytes");

static std::mutex g_scratch_mu;
static void* g_scratch_ptr[FA_NOALLOC_MAX_DEVICES];

// Device address of `scratch` on the stream's GPU (the current GPU for the
// null stream), looked up once per GPU with that GPU current.
static int scratch_for_stream(void* stream, void** out) {
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return FA_ERR_HIP;
  int dev = cur;
  if (stream && hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev) != hipSuccess) return FA_ERR_HIP;
  if (dev < 0 || dev >= FA_NOALLOC_MAX_DEVICES) return FA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return FA_ERR_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur && hipSetDevice(cur) != hipSuccess) return FA_ERR_HIP;
    if (e != hipSuccess || !p) return FA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return FA_OK;
}

int fa_backward_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                        const void* dout, void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale,
                        int causal, const int32_t* cu_seqlens, float dropout_p, uint64_t seed, void* stream,
                        int dtype, int64_t ld_qkv) {
  fa::AttnShape s;
  int rc = check_backward(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, d, scale, causal, cu_seqlens, dropout_p, seed,
                          dtype, ld_qkv, nullptr, false, &s);
  if (rc != FA_OK) return rc;
  if ((uint64_t)B * (uint64_t)N * (uint64_t)H > (uint64_t)FA_NOALLOC_MAX_ROWS) return FA_ERR_SCRATCH_LIMIT;
  void* ws = nullptr;
  if ((rc = scratch_for_stream(stream, &ws)) != FA_OK) return rc;
  return launch_backward_ws(s, fa::kBwdAll, q, k, v, o, lse, dout, dq, dk, dv, ws, stream);
}

size_t fa_decode_workspace_size(int B, int H, int nq, int nk_max, int d) {
  if (B < 1 || H < 1 || nq < 1 || nk_max < 1 || d < 1) return 0;
  const uint64_t rows = (uint64_t)B * (uint64_t)H * (uint64_t)fa::decode_splits(nk_max) * (uint64_t)nq;
  const uint64_t floats = rows * ((uint64_t)d + 2);
  if (floats > (UINT64_MAX / 8)) return 0;
  return (size_t)(floats * 4);
}

int fa_decode(const void* q, const void* k_cache, const void* v_cache, const int32_t* seqlens_k, void* o, float* lse,
              int B, int H, int nq, int nk_max, int d, float scale, int causal, void* stream, int dtype,
              void* workspace, size_t workspace_bytes) {
  if (!q || !k_cache || !v_cache || !o || !lse) return FA_ERR_NULL_POINTER;
  if (dtype != FA_DTYPE_F16 && dtype != FA_DTYPE_BF16) return FA_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (B < 1 || H < 1 || nq < 1 || nk_max < 1) return FA_ERR_BAD_SHAPE;
  if (nq > FA_DECODE_MAX_Q) return FA_ERR_UNSUPPORTED;
  if ((int64_t)B * H * fa::decode_splits(nk_max) > INT32_MAX || (int64_t)B * nq * H > INT32_MAX)
    return FA_ERR_BAD_SHAPE;
  if (!std::isfinite(scale) || !(scale > 0.f)) return FA_ERR_BAD_ARGUMENT;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o) || !aligned16(lse))
    return FA_ERR_ALIGNMENT;
  if (seqlens_k && (reinterpret_cast<uintptr_t>(seqlens_k) & 3u)) return FA_ERR_ALIGNMENT;
  const size_t need = fa_decode_workspace_size(B, H, nq, nk_max, d);
  if (!workspace || need == 0 || workspace_bytes < need) return FA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return FA_ERR_ALIGNMENT;
  fa::DecodeShape s{B, H, nq, nk_max, d, causal != 0, dtype == FA_DTYPE_BF16, scale};
  const hipError_t e = fa::launch_decode(s, q, k_cache, v_cache, seqlens_k, o, lse,
                                         static_cast<float*>(workspace), static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_decode_paged(const void* q, const void* k_pages, const void* v_pages, const int32_t* block_table,
                    const int32_t* seqlens_k, void* o, float* lse, int B, int H, int nq, int num_pages,
                    int page_size, int max_pages, int d, float scale, int causal, void* stream, int dtype,
                    void* workspace, size_t workspace_bytes) {
  if (!q || !k_pages || !v_pages || !block_table || !o || !lse) return FA_ERR_NULL_POINTER;
  if (dtype != FA_DTYPE_F16 && dtype != FA_DTYPE_BF16) return FA_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (B < 1 || H < 1 || nq < 1 || num_pages < 1 || max_pages < 1 || page_size < 1) return FA_ERR_BAD_SHAPE;
  if (page_size & (page_size - 1)) return FA_ERR_UNSUPPORTED;
  if (nq > FA_DECODE_MAX_Q) return FA_ERR_UNSUPPORTED;
  const int64_t capacity = (int64_t)max_pages * page_size;
  if (capacity > INT32_MAX || (int64_t)B * max_pages > INT32_MAX) return FA_ERR_BAD_SHAPE;
  const int nk_max = (int)capacity;
  if ((int64_t)B * H * fa::decode_splits(nk_max) > INT32_MAX || (int64_t)B * nq * H > INT32_MAX)
    return FA_ERR_BAD_SHAPE;
  if (!std::isfinite(scale) || !(scale > 0.f)) return FA_ERR_BAD_ARGUMENT;
  if (!aligned16(q) || !aligned16(k_pages) || !aligned16(v_pages) || !aligned16(o) || !aligned16(lse))
    return FA_ERR_ALIGNMENT;
  if (reinterpret_cast<uintptr_t>(block_table) & 3u) return FA_ERR_ALIGNMENT;
  if (seqlens_k && (reinterpret_cast<uintptr_t>(seqlens_k) & 3u)) return FA_ERR_ALIGNMENT;
  const size_t need = fa_decode_workspace_size(B, H, nq, nk_max, d);
  if (!workspace || need == 0 || workspace_bytes < need) return FA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return FA_ERR_ALIGNMENT;
  fa::DecodeShape s{B, H, nq, nk_max, d, causal != 0, dtype == FA_DTYPE_BF16, scale};
  const fa::DecodePages pages{block_table, page_size, max_pages, num_pages};
  const hipError_t e = fa::launch_decode(s, q, k_pages, v_pages, seqlens_k, o, lse, static_cast<float*>(workspace),
                                         static_cast<hipStream_t>(stream), &pages);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_dropout_mask(uint8_t* keep, int b, int h, int N, float dropout_p, uint64_t seed, void* stream) {
  if (!keep) return FA_ERR_NULL_POINTER;
  if (b < 0 || h < 0 || N < 1 || (int64_t)N * N > ((int64_t)1 << 40)) return FA_ERR_BAD_SHAPE;
  if (!(dropout_p >= 0.f) || !(dropout_p < 1.f)) return FA_ERR_BAD_ARGUMENT;
  const uint32_t t = (uint32_t)std::floor((double)dropout_p * 65536.0);
  const hipError_t e = fa::launch_dropout_mask(keep, b, h, N, t, seed, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

const char* fa_strerror(int code) {
  switch (code) {
    case FA_OK: return "success";
    case FA_ERR_NULL_POINTER: return "a required pointer is NULL";
    case FA_ERR_BAD_SHAPE: return "B, H and N must be >= 1 (and B*N tokens must fit in int32)";
    case FA_ERR_UNSUPPORTED: return "unsupported head dim (32, 64, 96, 128, 160, 192 or 256), dtype (fp16 or bf16), or length for block masks / stored keep bits";
    case FA_ERR_BAD_ARGUMENT: return "scale must be finite and > 0, dropout_p in [0, 1)";
    case FA_ERR_ALIGNMENT: return "pointers must be 16-byte aligned, ld_qkv a multiple of 8 and >= H*d";
    case FA_ERR_WORKSPACE: return "workspace (or keep-bit buffer) missing or smaller than fa_backward_workspace_size() (fa_dropout_bits_size())";
    case FA_ERR_HIP: return "a HIP kernel launch failed";
    case FA_ERR_SCRATCH_LIMIT: return "B*N*H exceeds FA_NOALLOC_MAX_ROWS, the fixed scratch of fa_backward_noalloc";
    default: return "unknown fa status code";
  }
}

}  // extern "C"
