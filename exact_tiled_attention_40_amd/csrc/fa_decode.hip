// KV-cache decode for gfx950 (MI355X): a few new query tokens per sequence
// attend to that sequence's cached keys and values (the inference-time cache
// use of the lab write-up "FlashAttention" (dpshk.com), section 6.1).
//
// The step reads every cached key and value once and does O(d) work per
// byte, so it is HBM-bound: no matrix cores, and the design is about keeping
// enough coalesced 16-byte loads in flight on every CU.
//   - Split-KV: one workgroup per (sequence, head, 1024-key chunk), so even a
//     single sequence fills the 256 CUs.  Lanes take 16-byte slices of key
//     rows (d/8 lanes per row), reduce the partial dot products across the
//     row with shuffles, and keep the chunk's scores in LDS; the chunk's max
//     and sum come from wave reductions; a second pass streams V and
//     accumulates P V per slice, reduced across row groups at the end.
//   - Each workgroup leaves its partial (O, m, l) in fp32 (m in log2 units);
//     the merge kernel combines the chunks of a query with the online-softmax
//     rule of section 3.2 of the lab write-up: M = max m, L = sum l 2^(m - M),
//     O = sum O_chunk 2^(m - M) / L, LSE = (M + log2 L) ln 2.
//   - A paged cache (page pools plus a block table) runs the same split
//     kernel with each chunk's page numbers staged in LDS first; only the row
//     addresses differ.
#include "fa_device.hpp"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kDecThreads = 256;
constexpr int kDecChunk = 1024;  // keys per split workgroup
constexpr int kDecBatch = 8;     // key rows each lane has in flight per tensor

struct DecArgs {
  const uint16_t* q;  // [B, nq, H, d]
  const uint16_t* k;  // [B, nk, H, d]
  const uint16_t* v;
  const int32_t* lk;  // [B] valid cache lengths, or nullptr (all nk)
  uint16_t* o;        // [B, nq, H, d]
  float* lse;         // [B, nq, H]
  float* part_o;      // [B*H, nsplit, nq, d]
  float* part_m;      // [B*H, nsplit, nq] (log2 units)
  float* part_l;      // [B*H, nsplit, nq]
  // paged cache: k and v are pools of num_pages pages of page_size tokens
  // ([num_pages, page_size, H, d]); cache position j of sequence b is token
  // j % page_size of page table[b * max_pages + j / page_size]
  const int32_t* table;
  int page_size, page_shift, max_pages, num_pages;
  int B, H, nq, nk, nsplit;
  float scale_log2;
};

template <bool BF16>
__device__ __forceinline__ void unpack8(u32x4 x, float (&f)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = to_f32<BF16>((uint16_t)(x[i] & 0xffff));
    f[2 * i + 1] = to_f32<BF16>((uint16_t)(x[i] >> 16));
  }
}

// Cache rows are read exactly once per step: non-temporal loads stream them
// past the caches instead of filling L2 and the memory-side cache with lines
// nothing reads again (measured 11 % faster on the 8 x 32 x 8192 cache).
__device__ __forceinline__ u32x4 load16(const uint16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

template <int D, bool BF16, bool CAUSAL, int NQ, bool PAGED>
__global__ __launch_bounds__(kDecThreads) void fa_decode_split_kernel(DecArgs a) {
  constexpr int kSl = D / 8;                // lanes per key row
  constexpr int kRows = kDecThreads / kSl;  // key rows per pass
  constexpr int kWv = kDecThreads / 64;
  static_assert(64 % kSl == 0, "a key row must lie within one wave");
  __shared__ float sc[NQ][kDecChunk];  // scores, then probabilities
  __shared__ float red[kWv][NQ][D];    // cross-wave sums of the P V slices
  __shared__ float wred[kWv][NQ];      // cross-wave max / sum

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int c = tid % kSl, g = tid / kSl;
  const int split = blockIdx.x % a.nsplit;
  const int bh = blockIdx.x / a.nsplit;
  const int b = bh / a.H, h = bh % a.H;
  const int L = a.lk ? min(max(a.lk[b], 0), a.nk) : a.nk;
  const int j0 = split * kDecChunk;
  const int n = max(0, min(L, j0 + kDecChunk) - j0);  // keys of this chunk
  const int nq = a.nq;
  const int64_t row = (int64_t)a.H * D;               // elements between tokens
  const int64_t base = PAGED ? 0 : ((int64_t)b * a.nk + j0) * row;
  const uint16_t* kb = a.k + base + (int64_t)h * D + 8 * c;
  const uint16_t* vb = a.v + base + (int64_t)h * D + 8 * c;
  // Paged: the chunk's page numbers, staged in LDS once so that no key load
  // waits on a table load; clamped into the pool, so every read stays in
  // bounds whatever the table holds.  Only the pages of the chunk's valid
  // keys are read from the table.
  __shared__ int pg[PAGED ? kDecChunk : 1];
  const int fp = PAGED ? j0 >> a.page_shift : 0;  // first page of the chunk
  if constexpr (PAGED) {
    const int npg = n > 0 ? ((j0 + n - 1) >> a.page_shift) - fp + 1 : 0;
    for (int i = tid; i < npg; i += kDecThreads)
      pg[i] = min(max(a.table[(int64_t)b * a.max_pages + fp + i], 0), a.num_pages - 1);
    __syncthreads();
  }
  // element offset of chunk row r (0 <= r < n) from kb / vb
  auto roff = [&](int r) __attribute__((always_inline)) -> int64_t {
    if constexpr (PAGED) {
      const int j = j0 + r;
      return ((int64_t)pg[(j >> a.page_shift) - fp] * a.page_size + (j & (a.page_size - 1))) * row;
    } else {
      return (int64_t)r * row;
    }
  };

  // this lane's slice of every query, prescaled by scale * log2(e)
  float qv[NQ][8];
#pragma unroll
  for (int t = 0; t < NQ; ++t) {
    if (t < nq) {
      unpack8<BF16>(load16(a.q + (((int64_t)b * nq + t) * a.H + h) * D + 8 * c), qv[t]);
#pragma unroll
      for (int e = 0; e < 8; ++e) qv[t][e] *= a.scale_log2;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) qv[t][e] = 0.f;
    }
  }

  // ---- pass 1: scores of the chunk into LDS (row r of the chunk: lanes
  // g == r % kRows)
  for (int r0 = 0; r0 < n; r0 += kRows * kDecBatch) {
    u32x4 kx[kDecBatch];
#pragma unroll
    for (int u = 0; u < kDecBatch; ++u) {
      const int r = r0 + u * kRows + g;
      kx[u] = r < n ? load16(kb + roff(r)) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kDecBatch; ++u) {
      const int r = r0 + u * kRows + g;
      float kf[8];
      unpack8<BF16>(kx[u], kf);
#pragma unroll
      for (int t = 0; t < NQ; ++t) {
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) s = __builtin_fmaf(qv[t][e], kf[e], s);
#pragma unroll
        for (int off = 1; off < kSl; off <<= 1) s += __shfl_xor(s, off, 64);
        if (c == 0 && r < n && t < nq) {
          const bool vis = !CAUSAL || j0 + r <= L - nq + t;
          sc[t][r] = vis ? s : -INFINITY;
        }
      }
    }
  }
  __syncthreads();

  // ---- chunk max and sum per query
  float m[NQ], l[NQ];
#pragma unroll
  for (int t = 0; t < NQ; ++t) {
    float x = -INFINITY;
    if (t < nq)
      for (int i = tid; i < n; i += kDecThreads) x = fmaxf(x, sc[t][i]);
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
    if (lane == 0) wred[w][t] = x;
  }
  __syncthreads();
#pragma unroll
  for (int t = 0; t < NQ; ++t) {
    float x = wred[0][t];
#pragma unroll
    for (int i = 1; i < kWv; ++i) x = fmaxf(x, wred[i][t]);
    m[t] = x;
  }
  __syncthreads();  // wred is reused below
#pragma unroll
  for (int t = 0; t < NQ; ++t) {
    float x = 0.f;
    if (t < nq && m[t] != -INFINITY)
      for (int i = tid; i < n; i += kDecThreads) {
        const float p = __builtin_amdgcn_exp2f(sc[t][i] - m[t]);
        sc[t][i] = p;
        x += p;
      }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) x += __shfl_xor(x, off, 64);
    if (lane == 0) wred[w][t] = x;
  }
  __syncthreads();
#pragma unroll
  for (int t = 0; t < NQ; ++t) {
    float x = 0.f;
#pragma unroll
    for (int i = 0; i < kWv; ++i) x += wred[i][t];
    l[t] = x;
  }

  // ---- pass 2: P V over the chunk, per 16-byte slice of V
  float acc[NQ][8];
#pragma unroll
  for (int t = 0; t < NQ; ++t)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[t][e] = 0.f;
  for (int r0 = 0; r0 < n; r0 += kRows * kDecBatch) {
    u32x4 vx[kDecBatch];
#pragma unroll
    for (int u = 0; u < kDecBatch; ++u) {
      const int r = r0 + u * kRows + g;
      vx[u] = r < n ? load16(vb + roff(r)) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kDecBatch; ++u) {
      const int r = r0 + u * kRows + g;
      if (r < n) {
        float vf[8];
        unpack8<BF16>(vx[u], vf);
#pragma unroll
        for (int t = 0; t < NQ; ++t) {
          const float p = (t < nq && m[t] != -INFINITY) ? sc[t][r] : 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[t][e] = __builtin_fmaf(p, vf[e], acc[t][e]);
        }
      }
    }
  }
  // reduce over the row groups: first inside the wave (lanes kSl apart hold
  // the same slice), then across waves through LDS
#pragma unroll
  for (int t = 0; t < NQ; ++t)
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int off = kSl; off < 64; off <<= 1) acc[t][e] += __shfl_xor(acc[t][e], off, 64);
  if (lane < kSl)
#pragma unroll
    for (int t = 0; t < NQ; ++t)
#pragma unroll
      for (int e = 0; e < 8; ++e) red[w][t][8 * c + e] = acc[t][e];
  __syncthreads();
  const int64_t pbase = ((int64_t)bh * a.nsplit + split) * nq;
  for (int i = tid; i < nq * D; i += kDecThreads) {
    const int t = i / D, dd = i % D;
    float x = 0.f;
#pragma unroll
    for (int ww = 0; ww < kWv; ++ww) x += red[ww][t][dd];
    a.part_o[(pbase + t) * D + dd] = x;
  }
  // every thread holds the chunk's m and l of every query; thread t writes query t's
#pragma unroll
  for (int t = 0; t < NQ; ++t)
    if (t == tid && t < nq) {
      a.part_m[pbase + t] = m[t];
      a.part_l[pbase + t] = l[t];
    }
}

// One wave per (sequence, query, head): combines the chunks' partial results.
template <int D, bool BF16>
__global__ __launch_bounds__(64) void fa_decode_merge_kernel(DecArgs a) {
  constexpr int kE = D / 64;  // output elements per lane
  const int lane = threadIdx.x;
  const int id = blockIdx.x;  // ((b * nq) + t) * H + h
  const int h = id % a.H;
  const int bt = id / a.H;
  const int t = bt % a.nq;
  const int b = bt / a.nq;
  const int64_t bh = (int64_t)b * a.H + h;
  float M = -INFINITY;
  for (int s = lane; s < a.nsplit; s += 64) M = fmaxf(M, a.part_m[(bh * a.nsplit + s) * a.nq + t]);
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
  float Lsum = 0.f, o[kE];
#pragma unroll
  for (int e = 0; e < kE; ++e) o[e] = 0.f;
  if (M != -INFINITY) {
    // a chunk with no visible key has m = -inf, l = 0 and O = 0: weight 0
#pragma unroll 4
    for (int s = 0; s < a.nsplit; ++s) {
      const int64_t p = (bh * a.nsplit + s) * a.nq + t;
      const float f = __builtin_amdgcn_exp2f(a.part_m[p] - M);
      Lsum += a.part_l[p] * f;
#pragma unroll
      for (int e = 0; e < kE; ++e) o[e] += a.part_o[p * D + lane + 64 * e] * f;
    }
  }
  const float inv = Lsum > 0.f ? 1.f / Lsum : 0.f;
  uint16_t* op = a.o + (((int64_t)b * a.nq + t) * a.H + h) * D;
#pragma unroll
  for (int e = 0; e < kE; ++e) {
    const uint32_t pk = pack2<BF16>(o[e] * inv, 0.f);
    op[lane + 64 * e] = (uint16_t)(pk & 0xffff);
  }
  if (lane == 0) a.lse[((int64_t)b * a.nq + t) * a.H + h] = Lsum > 0.f ? (M + log2f(Lsum)) * kLn2 : -INFINITY;
}

template <int D, bool BF16, bool CAUSAL, int NQ>
hipError_t launch_dec_q(const DecArgs& a, hipStream_t stream) {
  const int64_t nsplitwg = (int64_t)a.B * a.H * a.nsplit;
  const int64_t nmerge = (int64_t)a.B * a.nq * a.H;
  if (nsplitwg > 0x7fffffff || nmerge > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (a.table)
    hipLaunchKernelGGL((fa_decode_split_kernel<D, BF16, CAUSAL, NQ, true>), dim3((unsigned)nsplitwg),
                       dim3(kDecThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((fa_decode_split_kernel<D, BF16, CAUSAL, NQ, false>), dim3((unsigned)nsplitwg),
                       dim3(kDecThreads), 0, stream, a);
  hipLaunchKernelGGL((fa_decode_merge_kernel<D, BF16>), dim3((unsigned)nmerge), dim3(64), 0, stream, a);
  return hipGetLastError();
}

template <int D, bool BF16, bool CAUSAL>
hipError_t launch_dec_c(const DecArgs& a, hipStream_t stream) {
  if (a.nq == 1) return launch_dec_q<D, BF16, CAUSAL, 1>(a, stream);
  if (a.nq == 2) return launch_dec_q<D, BF16, CAUSAL, 2>(a, stream);
  if (a.nq <= 4) return launch_dec_q<D, BF16, CAUSAL, 4>(a, stream);
  return launch_dec_q<D, BF16, CAUSAL, 8>(a, stream);
}

template <int D, bool BF16>
hipError_t launch_dec_d(const DecodeShape& s, const DecArgs& a, hipStream_t stream) {
  return s.causal ? launch_dec_c<D, BF16, true>(a, stream) : launch_dec_c<D, BF16, false>(a, stream);
}

}  // namespace

int decode_splits(int nk) { return (nk + kDecChunk - 1) / kDecChunk; }

hipError_t launch_decode(const DecodeShape& s, const void* q, const void* k, const void* v, const int32_t* lk,
                         void* o, float* lse, float* workspace, hipStream_t stream, const DecodePages* pages) {
  DecArgs a;
  a.table = pages ? pages->table : nullptr;
  a.page_size = pages ? pages->page_size : 1;
  a.page_shift = pages ? __builtin_ctz((unsigned)pages->page_size) : 0;
  a.max_pages = pages ? pages->max_pages : 0;
  a.num_pages = pages ? pages->num_pages : 0;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.lk = lk;
  a.o = static_cast<uint16_t*>(o);
  a.lse = lse;
  a.B = s.B;
  a.H = s.H;
  a.nq = s.nq;
  a.nk = s.nk;
  a.nsplit = decode_splits(s.nk);
  const int64_t rows = (int64_t)s.B * s.H * a.nsplit * s.nq;
  a.part_o = workspace;
  a.part_m = workspace + rows * s.d;
  a.part_l = a.part_m + rows;
  a.scale_log2 = s.scale * kLog2e;
  if (s.d == 64)
    return s.bf16 ? launch_dec_d<64, true>(s, a, stream) : launch_dec_d<64, false>(s, a, stream);
  return s.bf16 ? launch_dec_d<128, true>(s, a, stream) : launch_dec_d<128, false>(s, a, stream);
}

}  // namespace fa
