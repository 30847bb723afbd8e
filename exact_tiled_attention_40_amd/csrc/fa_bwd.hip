// Exact attention backward for gfx950 (MI355X), recomputing P from the
// saved log-sum-exp instead of reading a stored P (lab write-up
// "FlashAttention" (dpshk.com), section 3.3).  Three kernels on one stream:
//
//   fa_bwd_pre   D[t][h] = sum_c dO[t][h][c] * O[t][h][c] (fp32) and zero the
//                fp32 dQ accumulator rows.  HBM-bound.
//   fa_bwd_main  one workgroup per (b, h, block of 128 keys); wave w owns
//                keys 32w .. 32w+31 with K and V of those keys in registers.
//                For every block of 64 queries that can see the keys:
//                  S  = Q K^T                 (MFMA, Q from LDS)
//                  P  = exp(S*scale - LSE)    (causal mask -> 0)
//                  dP = dO V^T                (MFMA, dO from LDS)
//                  dS = P * (dP - D)          (dropout: dP scaled by keep/(1-p))
//                  dV += Z^T dO, dK += dS^T Q (MFMA; Z^T and dS^T straight from
//                                              the accumulator registers, dO
//                                              and Q through LDS transpose reads)
//                  dQacc += dS K              (dS staged in LDS, fp32 atomics)
//   fa_bwd_dq    dQ = scale * dQacc -> bf16/fp16.
//
// The accumulator layout of S = Q K^T puts one key per lane and runs of four
// consecutive queries in registers, which is exactly the A-operand layout of
// the dV and dK products once the query order inside each 16-query MFMA
// slice is permuted (dO and Q are read with the same permutation).
#include "fa_device.hpp"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBKV = 32 * kWaves;  // keys per workgroup
constexpr int kBQ = 64;            // queries per inner iteration

template <int D>
struct BwdTile {
  static constexpr int kRow = D + 8;          // padded LDS row (16-bit elements) of Q, dO, K
  static constexpr int kDsRow = kBQ + 8;      // padded LDS row of dS^T ([key][query])
  static constexpr int kChunksPerRow = D / 8;
  static constexpr int kLoads = kBQ * kChunksPerRow / kThreads;  // 16-byte loads per thread per tensor
};

struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const float* lse;
  const uint16_t* dout;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  float* dq_acc;
  float* delta;
  const int32_t* cu;
  int64_t ld;
  int B, H, N, nkb;
  float scale;
  float scale_log2;
  uint32_t drop_thresh;
  float drop_rescale;
  uint32_t seed_lo, seed_hi;
};

__device__ __forceinline__ void seq_range(const BwdArgs& a, int b, int& start, int& L) {
  if (a.cu) {
    start = a.cu[b];
    L = a.cu[b + 1] - start;
  } else {
    start = b * a.N;
    L = a.N;
  }
}

// ---------------------------------------------------------------- preprocess
// D/8 lanes per (token, head) row; each lane owns 8 consecutive elements.
template <int D, bool BF16>
__global__ __launch_bounds__(256) void fa_bwd_pre_kernel(BwdArgs a) {
  constexpr int kLanesPerRow = D / 8;
  constexpr int kRowsPerBlock = 256 / kLanesPerRow;
  const int total = a.cu ? a.cu[a.B] : a.B * a.N;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / kLanesPerRow;
  const int c = (threadIdx.x % kLanesPerRow) * 8;
  const bool valid = row < (int64_t)total * a.H;
  float s = 0.f;
  if (valid) {
    const u32x4 o4 = *reinterpret_cast<const u32x4*>(a.o + row * D + c);
    const u32x4 g4 = *reinterpret_cast<const u32x4*>(a.dout + row * D + c);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      s += to_f32<BF16>((uint16_t)(o4[e] & 0xffff)) * to_f32<BF16>((uint16_t)(g4[e] & 0xffff));
      s += to_f32<BF16>((uint16_t)(o4[e] >> 16)) * to_f32<BF16>((uint16_t)(g4[e] >> 16));
    }
    float* acc = a.dq_acc + row * D + c;
    *reinterpret_cast<f32x4*>(acc) = f32x4{0.f, 0.f, 0.f, 0.f};
    *reinterpret_cast<f32x4*>(acc + 4) = f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int off = kLanesPerRow / 2; off > 0; off >>= 1) s += __shfl_xor(s, off, kLanesPerRow);
  if (valid && (threadIdx.x % kLanesPerRow) == 0) a.delta[row] = s;
}

// ---------------------------------------------------------------- main
template <int D, bool BF16, bool CAUSAL, bool DROPOUT>
__global__ __launch_bounds__(kThreads) void fa_bwd_main_kernel(BwdArgs a) {
  using T = BwdTile<D>;
  __shared__ __attribute__((aligned(16))) uint16_t q_s[kBQ * T::kRow];
  __shared__ __attribute__((aligned(16))) uint16_t do_s[kBQ * T::kRow];
  __shared__ __attribute__((aligned(16))) uint16_t k_s[kBKV * T::kRow];
  __shared__ __attribute__((aligned(16))) uint16_t ds_s[kBKV * T::kDsRow];
  __shared__ __attribute__((aligned(16))) float lse_s[kBQ];
  __shared__ __attribute__((aligned(16))) float dl_s[kBQ];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int h2 = lane >> 5;
  const int l32 = lane & 31;
  const int grp = lane >> 4;
  const int sl = lane & 15;
  const int c0 = 16 * (grp & 1);

  // Workgroup -> (b, h, key block); heads fastest (one head's blocks share an
  // XCD when B*H is a multiple of 8).  Causal: the first key blocks see the
  // most queries and go first.
  const int BH = a.B * a.H;
  const int bh = blockIdx.x % BH;
  const int kb = blockIdx.x / BH;
  const int b = bh / a.H;
  const int h = bh % a.H;
  int start, L;
  seq_range(a, b, start, L);
  const int j0 = kb * kBKV;
  if (j0 >= L) return;

  const int64_t ld = a.ld;
  const int64_t hoff = (int64_t)h * D;
  const int kw0 = j0 + 32 * w;   // first key of this wave
  const int kj = kw0 + l32;      // key owned by this lane

  // K, V fragments of this lane's key (B operand of Q K^T and dO V^T).
  u32x4 kf[D / 16], vf[D / 16];
  {
    const uint16_t* kp = a.k + (int64_t)(start + kj) * ld + hoff + 8 * h2;
    const uint16_t* vp = a.v + (int64_t)(start + kj) * ld + hoff + 8 * h2;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      kf[s] = kj < L ? *reinterpret_cast<const u32x4*>(kp + 16 * s) : u32x4{0, 0, 0, 0};
      vf[s] = kj < L ? *reinterpret_cast<const u32x4*>(vp + 16 * s) : u32x4{0, 0, 0, 0};
    }
  }
  // K block in LDS (B operand of dS K, read transposed).
  {
    constexpr int kKLoads = kBKV * T::kChunksPerRow / kThreads;
#pragma unroll
    for (int u = 0; u < kKLoads; ++u) {
      const int c = tid + kThreads * u;
      const int row = c / T::kChunksPerRow;
      const int col = (c % T::kChunksPerRow) * 8;
      u32x4 x = u32x4{0, 0, 0, 0};
      if (j0 + row < L) x = *reinterpret_cast<const u32x4*>(a.k + (int64_t)(start + j0 + row) * ld + hoff + col);
      *reinterpret_cast<u32x4*>(&k_s[row * T::kRow + col]) = x;
    }
  }

  f32x16 dv_acc[D / 32], dk_acc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
    dv_acc[dt] = f32x16{};
    dk_acc[dt] = f32x16{};
  }

  // Query blocks that can see this key block.
  const int i_begin = CAUSAL ? (j0 / kBQ) * kBQ : 0;
  const int n_iter = (L - i_begin + kBQ - 1) / kBQ;

  u32x4 qreg[T::kLoads], oreg[T::kLoads];
  float lse_r = 0.f, dl_r = 0.f;
  auto gload = [&](int i0) {
#pragma unroll
    for (int u = 0; u < T::kLoads; ++u) {
      const int c = tid + kThreads * u;
      const int row = c / T::kChunksPerRow;
      const int col = (c % T::kChunksPerRow) * 8;
      if (i0 + row < L) {
        qreg[u] = *reinterpret_cast<const u32x4*>(a.q + (int64_t)(start + i0 + row) * ld + hoff + col);
        oreg[u] = *reinterpret_cast<const u32x4*>(a.dout + (int64_t)(start + i0 + row) * a.H * D + hoff + col);
      } else {
        qreg[u] = u32x4{0, 0, 0, 0};
        oreg[u] = u32x4{0, 0, 0, 0};
      }
    }
    if (tid < kBQ) {
      const int i = i0 + tid;
      // rows past the end get LSE = +inf so that P = 0 there
      lse_r = i < L ? a.lse[(int64_t)(start + i) * a.H + h] * kLog2e : INFINITY;
      dl_r = i < L ? a.delta[(int64_t)(start + i) * a.H + h] : 0.f;
    }
  };
  auto sstore = [&]() {
#pragma unroll
    for (int u = 0; u < T::kLoads; ++u) {
      const int c = tid + kThreads * u;
      const int row = c / T::kChunksPerRow;
      const int col = (c % T::kChunksPerRow) * 8;
      *reinterpret_cast<u32x4*>(&q_s[row * T::kRow + col]) = qreg[u];
      *reinterpret_cast<u32x4*>(&do_s[row * T::kRow + col]) = oreg[u];
    }
    if (tid < kBQ) {
      lse_s[tid] = lse_r;
      dl_s[tid] = dl_r;
    }
  };

  if (n_iter > 0) gload(i_begin);
  for (int it = 0; it < n_iter; ++it) {
    const int i0 = i_begin + it * kBQ;
    sstore();
    __syncthreads();
    if (it + 1 < n_iter) gload(i0 + kBQ);

    const bool active = !CAUSAL || i0 + kBQ - 1 >= kw0;
    uint16_t* dsw = &ds_s[(32 * w + l32) * T::kDsRow];
    if (active) {
      // ---- S = Q K^T and dP = dO V^T for 64 queries x this wave's 32 keys
      f32x16 sacc[2], pacc[2];
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        sacc[qt] = f32x16{};
        pacc[qt] = f32x16{};
        const uint16_t* qp = &q_s[(qt * 32 + l32) * T::kRow + 8 * h2];
        const uint16_t* gp = &do_s[(qt * 32 + l32) * T::kRow + 8 * h2];
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
          sacc[qt] = mfma32<BF16>(lds_read16(qp + 16 * s), kf[s], sacc[qt]);
          pacc[qt] = mfma32<BF16>(lds_read16(gp + 16 * s), vf[s], pacc[qt]);
        }
      }
      // ---- P, dS (register r of tile qt: query qt*32 + 8*(r/4) + 4*h2 + r%4)
      const bool need_mask = CAUSAL && i0 < kw0 + 31;
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int qrow = qt * 32 + 8 * g + 4 * h2;
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(&lse_s[qrow]);
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(&dl_s[qrow]);
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int r = 4 * g + t;
            float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[qt][r], a.scale_log2, -l4[t]));
            if (need_mask && kj > i0 + qrow + t) p = 0.f;
            float dp = pacc[qt][r];
            float z = p;
            if constexpr (DROPOUT) {
              const uint32_t qi = (uint32_t)(i0 + qrow + t);
              const Philox4 rnd = philox4x32_10(qi, (uint32_t)kj >> 2, (uint32_t)h, (uint32_t)b, a.seed_lo,
                                                a.seed_hi);
              const uint32_t wsel = (kj & 3) == 0 ? rnd.x : (kj & 3) == 1 ? rnd.y : (kj & 3) == 2 ? rnd.z : rnd.w;
              const float kf_ = wsel >= a.drop_thresh ? a.drop_rescale : 0.f;
              dp *= kf_;
              z = p * kf_;
            }
            sacc[qt][r] = z;                  // Z (= P without dropout) for dV
            pacc[qt][r] = p * (dp - d4[t]);   // dS
          }
        }
      // ---- dV += Z^T dO, dK += dS^T Q over four 16-query slices
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int qt = m >> 1;
        const int sub = (m & 1) * 8;
        const u32x4 zf = {pack2<BF16>(sacc[qt][sub + 0], sacc[qt][sub + 1]),
                          pack2<BF16>(sacc[qt][sub + 2], sacc[qt][sub + 3]),
                          pack2<BF16>(sacc[qt][sub + 4], sacc[qt][sub + 5]),
                          pack2<BF16>(sacc[qt][sub + 6], sacc[qt][sub + 7])};
        const u32x4 sf = {pack2<BF16>(pacc[qt][sub + 0], pacc[qt][sub + 1]),
                          pack2<BF16>(pacc[qt][sub + 2], pacc[qt][sub + 3]),
                          pack2<BF16>(pacc[qt][sub + 4], pacc[qt][sub + 5]),
                          pack2<BF16>(pacc[qt][sub + 6], pacc[qt][sub + 7])};
        const int row = 16 * m + 4 * h2 + (sl >> 2);
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          const int col = dt * 32 + c0 + 4 * (sl & 3);
          const u32x2 g0 = lds_read_tr(&do_s[row * T::kRow + col]);
          const u32x2 g1 = lds_read_tr(&do_s[(row + 8) * T::kRow + col]);
          dv_acc[dt] = mfma32<BF16>(zf, u32x4{g0[0], g0[1], g1[0], g1[1]}, dv_acc[dt]);
          const u32x2 q0 = lds_read_tr(&q_s[row * T::kRow + col]);
          const u32x2 q1 = lds_read_tr(&q_s[(row + 8) * T::kRow + col]);
          dk_acc[dt] = mfma32<BF16>(sf, u32x4{q0[0], q0[1], q1[0], q1[1]}, dk_acc[dt]);
        }
        // dS^T row of this lane's key: four runs of 4 consecutive queries
      }
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const u32x2 pk = {pack2<BF16>(pacc[qt][4 * g + 0], pacc[qt][4 * g + 1]),
                            pack2<BF16>(pacc[qt][4 * g + 2], pacc[qt][4 * g + 3])};
          *reinterpret_cast<u32x2*>(dsw + qt * 32 + 8 * g + 4 * h2) = pk;
        }
    } else {
      // keys after every query of the block: dS = 0
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int g = 0; g < 4; ++g) *reinterpret_cast<u32x2*>(dsw + qt * 32 + 8 * g + 4 * h2) = u32x2{0, 0};
    }
    __syncthreads();

    // ---- dQacc[64 x D] += dS K over the 128 keys; wave w: query tile w&1,
    // head-dim tiles (w>>1)*NCT .. +NCT-1
    {
      constexpr int NCT = D / 64;
      const int qt = w & 1;
      f32x16 qacc[NCT];
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) qacc[ct] = f32x16{};
#pragma unroll
      for (int kk = 0; kk < kBKV / 16; ++kk) {
        const int krow = 16 * kk + 8 * h2 + (sl >> 2);
        const u32x2 a0 = lds_read_tr(&ds_s[krow * T::kDsRow + qt * 32 + c0 + 4 * (sl & 3)]);
        const u32x2 a1 = lds_read_tr(&ds_s[(krow + 4) * T::kDsRow + qt * 32 + c0 + 4 * (sl & 3)]);
        const u32x4 af = {a0[0], a0[1], a1[0], a1[1]};
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          const int col = ((w >> 1) * NCT + ct) * 32 + c0 + 4 * (sl & 3);
          const u32x2 b0 = lds_read_tr(&k_s[krow * T::kRow + col]);
          const u32x2 b1 = lds_read_tr(&k_s[(krow + 4) * T::kRow + col]);
          qacc[ct] = mfma32<BF16>(af, u32x4{b0[0], b0[1], b1[0], b1[1]}, qacc[ct]);
        }
      }
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const int c = ((w >> 1) * NCT + ct) * 32 + l32;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int i = i0 + qt * 32 + 8 * (r >> 2) + 4 * h2 + (r & 3);
          if (i < L) atomicAdd(a.dq_acc + ((int64_t)(start + i) * a.H + h) * D + c, qacc[ct][r]);
        }
      }
    }
    __syncthreads();
  }

  // ---- epilogue: dK = scale * dK_acc, dV; register r: key kw0 + 8*(r/4) + 4*h2 + r%4, lane: column
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int j = kw0 + 8 * (r >> 2) + 4 * h2 + (r & 3);
      if (j < L) {
        const int64_t off = (int64_t)(start + j) * ld + hoff + dt * 32 + l32;
        const uint32_t pk = pack2<BF16>(dk_acc[dt][r] * a.scale, dv_acc[dt][r]);
        a.dk[off] = (uint16_t)(pk & 0xffff);
        a.dv[off] = (uint16_t)(pk >> 16);
      }
    }
}

// ---------------------------------------------------------------- dQ convert
template <int D, bool BF16>
__global__ __launch_bounds__(256) void fa_bwd_dq_kernel(BwdArgs a) {
  const int total = a.cu ? a.cu[a.B] : a.B * a.N;
  const int64_t idx = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;  // element index in [tokens, H, D]
  if (idx >= (int64_t)total * a.H * D) return;
  const int64_t row = idx / D;          // token * H + head
  const int c = (int)(idx % D);
  const int64_t tok = row / a.H;
  const int hh = (int)(row % a.H);
  const f32x4 x0 = *reinterpret_cast<const f32x4*>(a.dq_acc + idx);
  const f32x4 x1 = *reinterpret_cast<const f32x4*>(a.dq_acc + idx + 4);
  const u32x4 pk = {pack2<BF16>(x0[0] * a.scale, x0[1] * a.scale), pack2<BF16>(x0[2] * a.scale, x0[3] * a.scale),
                    pack2<BF16>(x1[0] * a.scale, x1[1] * a.scale), pack2<BF16>(x1[2] * a.scale, x1[3] * a.scale)};
  *reinterpret_cast<u32x4*>(a.dq + tok * a.ld + (int64_t)hh * D + c) = pk;
}

template <int D, bool BF16>
hipError_t launch_bwd_d(const AttnShape& s, const BwdArgs& args, int stages, hipStream_t stream) {
  const int64_t rows = (int64_t)s.B * s.N * s.H;
  if (stages & kBwdPre) {
    constexpr int kRowsPerBlock = 256 / (D / 8);
    const int64_t nb = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
    if (nb > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((fa_bwd_pre_kernel<D, BF16>), dim3((unsigned)nb), dim3(256), 0, stream, args);
  }
  if (stages & kBwdMain) {
    const int64_t nb = (int64_t)args.nkb * s.B * s.H;
    if (nb > 0x7fffffff) return hipErrorInvalidConfiguration;
    auto kern = s.causal ? (s.dropout ? fa_bwd_main_kernel<D, BF16, true, true> : fa_bwd_main_kernel<D, BF16, true, false>)
                         : (s.dropout ? fa_bwd_main_kernel<D, BF16, false, true>
                                      : fa_bwd_main_kernel<D, BF16, false, false>);
    hipLaunchKernelGGL(kern, dim3((unsigned)nb), dim3(kThreads), 0, stream, args);
  }
  if (stages & kBwdDq) {
    const int64_t nb = (rows * D / 8 + 255) / 256;
    if (nb > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((fa_bwd_dq_kernel<D, BF16>), dim3((unsigned)nb), dim3(256), 0, stream, args);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_backward(const AttnShape& s, const void* q, const void* k, const void* v, const void* o,
                           const float* lse, const void* dout, void* dq, void* dk, void* dv, float* dq_acc,
                           float* delta, int stages, hipStream_t stream) {
  BwdArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<const uint16_t*>(o);
  a.lse = lse;
  a.dout = static_cast<const uint16_t*>(dout);
  a.dq = static_cast<uint16_t*>(dq);
  a.dk = static_cast<uint16_t*>(dk);
  a.dv = static_cast<uint16_t*>(dv);
  a.dq_acc = dq_acc;
  a.delta = delta;
  a.cu = s.cu;
  a.ld = s.ld;
  a.B = s.B;
  a.H = s.H;
  a.N = s.N;
  a.nkb = (s.N + kBKV - 1) / kBKV;
  a.scale = s.scale;
  a.scale_log2 = s.scale * kLog2e;
  a.drop_thresh = s.drop_thresh;
  a.drop_rescale = s.drop_rescale;
  a.seed_lo = (uint32_t)s.seed;
  a.seed_hi = (uint32_t)(s.seed >> 32);
  if (s.d == 64)
    return s.bf16 ? launch_bwd_d<64, true>(s, a, stages, stream) : launch_bwd_d<64, false>(s, a, stages, stream);
  return s.bf16 ? launch_bwd_d<128, true>(s, a, stages, stream) : launch_bwd_d<128, false>(s, a, stages, stream);
}

}  // namespace fa
