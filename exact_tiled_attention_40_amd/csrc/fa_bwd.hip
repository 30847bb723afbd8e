// Exact attention backward for gfx950 (MI355X), recomputing P from the
// saved log-sum-exp instead of reading a stored P (lab write-up
// "FlashAttention" (dpshk.com), section 3.3).  Two kernels on one stream;
// neither uses atomics:
//
//   fa_bwd_dq_kernel    one workgroup per (b, h, block of 256 queries), eight
//                       waves of 32 queries (block-sparse: 128 queries, four
//                       waves, one mask row).  Prologue: D = rowsum(dO * O)
//                       for its rows (kept in registers and written to the
//                       workspace).  For every 64-key tile the queries can
//                       see (K and V tiles double-buffered HBM -> LDS):
//                         S^T  = K Q^T              (MFMA, Q in registers)
//                         dP^T = V dO^T             (MFMA, dO in registers)
//                         P    = exp(S*scale - LSE)  (masked -> 0)
//                         dS   = P * (dP - D)        (dropout: dP * keep/(1-p))
//                         dQ^T += K^T dS^T           (MFMA, fp32 accumulator in
//                                                     registers, K^T through the
//                                                     LDS transpose read)
//                       Epilogue: dQ = scale * dQ, rounded once.
//   fa_bwd_dkdv_kernel  one workgroup per (b, h, block of 128 keys), four
//                       waves of 32 keys whose K and V stay in registers.
//                       For every 64-query tile that can see the keys (Q, dO,
//                       LSE and D tiles double-buffered HBM -> LDS):
//                         S  = Q K^T, dP = dO V^T   (MFMA, Q and dO from LDS)
//                         P, Z = P * keep/(1-p), dS = P * (dP - D)
//                         dV += Z^T dO, dK += dS^T Q (MFMA; Z^T and dS^T straight
//                                                    from the accumulator
//                                                    registers, dO and Q through
//                                                    the LDS transpose read)
//                       Epilogue: dK = scale * dK; dK, dV rounded once.
//
// Both kernels recompute S and dP (two extra products per visible pair) so
// that dQ, dK and dV each have one owner: an fp32 atomic reduction of dQ over
// key blocks would move more bytes through the atomic units than the rest of
// the backward moves through HBM, while the recomputation runs on the matrix
// cores.  The dQ kernel runs first because the dK/dV kernel reads its D.
#include <type_traits>

#include "fa_device.hpp"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kWaves = 4;          // dK/dV kernel: one wave per SIMD
constexpr int kThreads = 64 * kWaves;
// dQ kernel: dense with heads up to 128, eight waves (two per SIMD, one
// workgroup per CU), so each K/V tile in LDS serves 256 queries;
// block-sparse, four waves (128 queries, one mask row, so the tile list is
// exact) and two workgroups per CU; heads above 128, four waves with one
// workgroup per CU (the Q, dO fragments and the dQ accumulator of a wave
// need more than half the register file).
template <bool SPARSE, int D> constexpr int dq_waves() { return (SPARSE || D > 128) ? 4 : 8; }
template <bool SPARSE, int D> constexpr int dq_rows() { return 32 * dq_waves<SPARSE, D>(); }
template <bool SPARSE, int D> constexpr int dq_wgs_per_cu() { return (SPARSE && D <= 128) ? 2 : 1; }
constexpr int kBC = 64;            // keys per tile of the dQ kernel
constexpr int kBKV = 32 * kWaves;  // keys per dK/dV workgroup
constexpr int kBR = 64;            // queries per tile of the dK/dV kernel
constexpr int kKvHeadGroup = 2;    // dK/dV kernel: heads an XCD works on at a time

// Instruction classes of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedValu = 0x2, kSchedMfma = 0x8, kSchedDsRead = 0x100;

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
  float* delta;   // D = rowsum(dO * O), [tokens, H]
  float* lse2;    // LSE * log2(e), [tokens, H]
  const int32_t* cu;
  const uint32_t* kbits;  // keep-bit instantiations only: the forward's decisions (layout: fa_internal.h)
  int nkt;                // ceil(N / 64)
  int kbn;                // row stride of the keep-bit planes (N rounded up to 4)
  int64_t ld;
  int B, H, N, nqb, nkb;
  float scale;
  float scale_log2;
  uint32_t drop_thresh;
  float drop_rescale;
  uint32_t seed_lo, seed_hi;
  const uint8_t* bmask;  // block-sparse instantiations only: [B, H, nb, nb]
  int nb;
};

__device__ __forceinline__ void seq_range(const BwdArgs& a, int b, int& start, int& L) {
  seq_bounds(a.cu, b, a.B, a.N, start, L);
}

// ---------------------------------------------------------------- dQ (+ D)
template <int D, bool BF16, bool CAUSAL, bool DROPOUT, bool SPARSE, bool KB = false>
__global__ __launch_bounds__((64 * dq_waves<SPARSE, D>()), (dq_wgs_per_cu<SPARSE, D>())) void fa_bwd_dq_kernel(
    BwdArgs a) {
  static_assert(!KB || (DROPOUT && !SPARSE), "keep bits: dense dropout instantiations only");
  static_assert(!KB || kBC == 64, "keep-bit words cover 64-key tiles");
  using T = MTile<D, kBC>;
  constexpr int kWavesQ = dq_waves<SPARSE, D>();
  constexpr int kBQ = dq_rows<SPARSE, D>();
  constexpr int kNS = 2 * (D / 16);  // S^T and dP^T products per 32-key half (D/16 k-steps each)
  constexpr int kNQ = 2 * (D / 32);  // dQ^T products per 32-key half (two 16-key slices x D/32 tiles)
  constexpr int kPF = 2;             // LDS operand reads in flight (products ahead)
  __shared__ __attribute__((aligned(1024))) uint16_t ks[2][T::kElems];
  __shared__ __attribute__((aligned(1024))) uint16_t vs[2][T::kElems];
  // keep bits: the stored words of the workgroup's queries against the key
  // tile of the buffer, two planes (keys 0-31, 32-63 of the tile) of kBQ rows
  __shared__ __attribute__((aligned(1024))) uint32_t kbs[KB ? 2 : 1][KB ? 2 * kBQ : 4];
  // block-sparse: the key tiles the workgroup visits, in order
  __shared__ uint16_t tlist[SPARSE ? kMaxSparseTiles : 1];
  __shared__ uint8_t tflag[SPARSE ? kMaxSparseTiles : 1];
  __shared__ int tcount[1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h2 = lane >> 5;
  const int l32 = lane & 31;

  // Workgroup -> (b, h, query block): heads fastest (one head's blocks share
  // an XCD when B*H is a multiple of 8); causal: longest blocks first.  (Two
  // heads at a time per XCD cut the fetched bytes at B 4, H 8, N 4096, d 128
  // causal from 279 to 234 MB but ran 1.4% slower.)
  const int BH = a.B * a.H;
  const int bh = blockIdx.x % BH;
  const int rank = blockIdx.x / BH;
  const int b = bh / a.H;
  const int h = bh % a.H;
  const int qb = CAUSAL ? a.nqb - 1 - rank : rank;
  int start, L;
  seq_range(a, b, start, L);
  const int q0 = qb * kBQ;
  if (q0 >= L) return;

  const int64_t ld = a.ld;
  const int64_t hd = (int64_t)a.H * D;  // token stride of o, dout
  const uint32_t row_bytes = (uint32_t)ld * 2;
  const uint16_t* kbase = a.k + (int64_t)start * ld + (int64_t)h * D;
  const uint16_t* vbase = a.v + (int64_t)start * ld + (int64_t)h * D;
  const int kv_end = CAUSAL ? min(L, q0 + kBQ) : L;
  const int ntiles = (kv_end + kBC - 1) / kBC;

  const int qw = q0 + 32 * w;
  const int qi = qw + l32;

  // Q and dO fragments (B operands: column = query, K slice = head dim) and
  // D = rowsum(dO * O) of this lane's query; rows past the end read as zeros.
  u32x4 qf[D / 16], gf[D / 16];
  float delta;
  {
    const int rows = max(0, min(32, L - qw));
    const int64_t tok = start + min(qw, L - 1);
    const __amdgpu_buffer_rsrc_t qr =
        make_rsrc(a.q + tok * ld + (int64_t)h * D, rows > 0 ? (uint32_t)(rows - 1) * row_bytes + D * 2 : 0u);
    const uint32_t gbytes = rows > 0 ? (uint32_t)(rows - 1) * (uint32_t)hd * 2 + D * 2 : 0u;
    const __amdgpu_buffer_rsrc_t gr = make_rsrc(a.dout + tok * hd + (int64_t)h * D, gbytes);
    const __amdgpu_buffer_rsrc_t orr = make_rsrc(a.o + tok * hd + (int64_t)h * D, gbytes);
    const uint32_t offq = (uint32_t)l32 * row_bytes + 16 * h2;
    const uint32_t offg = (uint32_t)l32 * (uint32_t)hd * 2 + 16 * h2;
    u32x4 of[D / 16];
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      qf[s] = buffer_load16(qr, offq + 32 * s);
      gf[s] = buffer_load16(gr, offg + 32 * s);
      of[s] = buffer_load16(orr, offg + 32 * s);
    }
    float acc = 0.f;
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc += to_f32<BF16>((uint16_t)(gf[s][e] & 0xffff)) * to_f32<BF16>((uint16_t)(of[s][e] & 0xffff));
        acc += to_f32<BF16>((uint16_t)(gf[s][e] >> 16)) * to_f32<BF16>((uint16_t)(of[s][e] >> 16));
      }
    delta = halves_sum(acc);
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      asm volatile("" : "+v"(qf[s]));
      asm volatile("" : "+v"(gf[s]));
    }
  }
  // queries past the end: Q = dO = 0 and LSE = 0 give P = 1, dP = 0, dS = 0.
  // A query that sees no key (block-sparse) has LSE = -inf; +inf in its place
  // makes every P of the row 0 wherever it is recomputed.
  float lse2 = qi < L ? a.lse[(int64_t)(start + qi) * a.H + h] * kLog2e : 0.f;
  if constexpr (SPARSE) lse2 = lse2 == -INFINITY ? INFINITY : lse2;
  if (qi < L && h2 == 0) {
    a.delta[(int64_t)(start + qi) * a.H + h] = delta;
    a.lse2[(int64_t)(start + qi) * a.H + h] = lse2;
  }

  const uint32_t ks0 = lds_addr(ks), vs0 = lds_addr(vs);
  // the stored keep words of this head (at most 512 MB: N <= 65536)
  const __amdgpu_buffer_rsrc_t kbr =
      KB ? make_rsrc(a.kbits + (int64_t)bh * a.nkt * 2 * a.kbn, (uint32_t)((uint64_t)a.nkt * 2 * a.kbn * 4))
         : make_rsrc(nullptr, 0u);
  auto issue_tile = [&](int j0, int buf) {
    const int rows = min(kBC, L - j0);
    const uint32_t bytes = (uint32_t)(rows - 1) * row_bytes + D * 2;
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(kbase + (int64_t)j0 * ld, bytes);
    const __amdgpu_buffer_rsrc_t vr = make_rsrc(vbase + (int64_t)j0 * ld, bytes);
    if constexpr (KB) {
      // 8 * kBQ bytes of stored words: 1 KB loads by the first kBQ / 128
      // waves; lane l of load m takes the 16 bytes at m * 1024 + 16 l of the
      // two planes laid end to end (rows past the head's buffer read as 0)
      static_assert(kBQ % 128 == 0 && kBQ / 128 <= kWavesQ, "keep-bit loads");
      if (w < kBQ / 128) {
        const uint32_t f = (uint32_t)w * 1024 + 16 * lane;
        const uint32_t plane = f / (4 * kBQ), r = (f % (4 * kBQ)) / 4;
        const int t = j0 / kBC;
        const uint32_t word = ((uint32_t)t * 2 + plane) * (uint32_t)a.kbn + (uint32_t)q0 + r;
        buffer_load_lds16_addr(kbr, lds_addr(kbs[buf]) + (uint32_t)w * 1024, word * 4);
      }
    }
    // wave w loads blocks w, w + kWavesQ, ... (a partial last round when
    // the tile has fewer blocks than a multiple of the waves)
#pragma unroll
    for (int u = 0; u < (T::kBlocks + kWavesQ - 1) / kWavesQ; ++u) {
      if (u * kWavesQ + w < T::kBlocks) {
        T::load(kr, ks0 + buf * T::kBytes, row_bytes, u * kWavesQ + w, lane);
        T::load(vr, vs0 + buf * T::kBytes, row_bytes, u * kWavesQ + w, lane);
      }
    }
  };

  f32x16 qacc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) qacc[dt] = f32x16{};

  const uint32_t ob0 = T::opnd_base(lane, 0), ob1 = T::opnd_base(lane, 1);
  const uint32_t tb0 = T::tr_base(lane, 0), tb1 = T::tr_base(lane, 1);

  // Visited key tiles: all tiles 0 .. ntiles-1, or (block-sparse) the listed
  // ones.  Buffers follow the position k in that sequence; tile_at(k) is the
  // tile index.
  int n_list = ntiles;
  if constexpr (SPARSE) {
    if (w == 0) {
      static_assert(!SPARSE || kBQ == kMaskBlock, "one mask row per block-sparse workgroup");
      const uint8_t* mrow = a.bmask + (((int64_t)b * a.H + h) * a.nb + q0 / kMaskBlock) * a.nb;
      const int n = build_tile_list(mrow, nullptr, 0, 1, ntiles, tlist, tflag, lane);
      if (lane == 0) tcount[0] = n;
    }
    __syncthreads();
    n_list = __builtin_amdgcn_readfirstlane(tcount[0]);
  }
  auto tile_at = [&](int k) __attribute__((always_inline)) -> int {
    if constexpr (SPARSE) return __builtin_amdgcn_readfirstlane(tlist[k]);
    else return k;
  };

  if (n_list > 0) issue_tile(tile_at(0) * kBC, 0);
  wait_vmem();
  __syncthreads();

  // One tile of 64 keys, as two 32-key halves kt.  Per half, in a fixed
  // order (sched_barrier fences keep it): S^T = K Q^T and dP^T = V dO^T
  // interleaved, their K/V operands read kPF products ahead; the first K^T
  // transpose reads; P and dS; dQ^T += K^T dS^T with its K^T operands read
  // kPF products ahead.
  auto tile = [&](int k, int t, auto mask_tag) __attribute__((always_inline)) {  // position k, tile t
    constexpr bool kMask = decltype(mask_tag)::value;
    const int cur = k & 1;
    const int j0 = t * kBC;
    uint32_t k0 = ks0 + cur * T::kBytes + ob0, k1 = ks0 + cur * T::kBytes + ob1;
    uint32_t v0 = vs0 + cur * T::kBytes + ob0, v1 = vs0 + cur * T::kBytes + ob1;
    uint32_t kt0 = ks0 + cur * T::kBytes + tb0, kt1 = ks0 + cur * T::kBytes + tb1;
    asm volatile("" : "+v"(k0), "+v"(k1), "+v"(v0), "+v"(v1), "+v"(kt0), "+v"(kt1));
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      // product i: tensor i & 1 (K for S, V for dP), k-step i >> 1
      auto sread = [&](int i) {
        const int s = i >> 1;
        const uint32_t base = (i & 1) ? ((s & 1) ? v1 : v0) : ((s & 1) ? k1 : k0);
        return lds_read16_at(base + T::opnd_off(kt, s));
      };
      // product j: key slice 2kt + j / (D/32), head-dim tile j % (D/32)
      auto qread = [&](int j) {
        const uint32_t o = T::tr_off(2 * kt + j / (D / 32), j % (D / 32));
        const u32x2 lo = lds_read_tr_at(kt0 + o), hi = lds_read_tr_at(kt1 + o);
        return u32x4{lo[0], lo[1], hi[0], hi[1]};
      };
      f32x16 sacc = f32x16{}, pacc = f32x16{};
      u32x4 sb[kNS];
#pragma unroll
      for (int i = 0; i < kPF; ++i) sb[i] = sread(i);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < kNS; ++i) {
        if (i & 1)
          pacc = mfma32<BF16>(sb[i], gf[i >> 1], pacc);
        else
          sacc = mfma32<BF16>(sb[i], qf[i >> 1], sacc);
        if (i + kPF < kNS) sb[i + kPF] = sread(i + kPF);
        __builtin_amdgcn_sched_barrier(0);
      }
      u32x4 qb_[kNQ];
#pragma unroll
      for (int j = 0; j < kPF; ++j) qb_[j] = qread(j);

      // ---- P and dS; register r: key j0 + kt*32 + 8*(r/4) + 4*h2 + r%4
      uint32_t spk[8];
      // dropout: this lane's keep words of the four 8-key groups of the half
      uint32_t kw[2][2][2];  // [group pair][group of the pair][word]
      uint32_t kbw = 0;      // keep bits: key 8g + e of the lane's half at bit 8g + e
      if constexpr (DROPOUT && !KB) {
        keep_words_pair(qi, j0 + kt * 32, h2, h, b, a.seed_lo, a.seed_hi, kw[0]);
        keep_words_pair(qi, j0 + kt * 32 + 16, h2, h, b, a.seed_lo, a.seed_hi, kw[1]);
      }
      if constexpr (KB) kbw = kbs[cur][kt * kBQ + (qi - q0)] >> (4 * h2);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int kj4 = j0 + kt * 32 + 8 * g + 4 * h2;
        float ds[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g + e;
          float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[r], a.scale_log2, -lse2));
          if (kMask && ((CAUSAL && kj4 + e > qi) || kj4 + e >= L)) p = 0.f;
          float dp = pacc[r];
          if constexpr (KB)
            dp *= (kbw >> (8 * g + e)) & 1u ? a.drop_rescale : 0.f;
          else if constexpr (DROPOUT)
            dp *= keep16(kw[g >> 1][g & 1][e >> 1], e & 1, a.drop_thresh) ? a.drop_rescale : 0.f;
          ds[e] = p * (dp - delta);
        }
        spk[2 * g] = pack2<BF16>(ds[0], ds[1]);
        spk[2 * g + 1] = pack2<BF16>(ds[2], ds[3]);
      }
      const u32x4 sf[2] = {u32x4{spk[0], spk[1], spk[2], spk[3]}, u32x4{spk[4], spk[5], spk[6], spk[7]}};
      __builtin_amdgcn_sched_barrier(0);

      // ---- dQ^T += K^T dS^T over the two 16-key slices of this half
#pragma unroll
      for (int j = 0; j < kNQ; ++j) {
        qacc[j % (D / 32)] = mfma32<BF16>(qb_[j], sf[j / (D / 32)], qacc[j % (D / 32)]);
        if (j + kPF < kNQ) qb_[j + kPF] = qread(j + kPF);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // Last tile this wave needs (its queries all precede the later ones; a
  // wave past a ragged end needs none).  Only that tile can hold masked keys
  // (causal diagonal or the ragged end), so the tiles before it run without
  // mask code, and the loop keeps one accumulator path.  Every wave still
  // issues its share of every tile load and joins every barrier.
  const int last = qw >= L ? -1 : (CAUSAL ? min(ntiles - 1, (qw + 31) / kBC) : ntiles - 1);
  int k = 0;
  int tk = n_list > 0 ? tile_at(0) : -1;
  for (; k < n_list && tk < last; ++k) {
    const int tk1 = k + 1 < n_list ? tile_at(k + 1) : -1;
    if (tk1 >= 0) issue_tile(tk1 * kBC, (k & 1) ^ 1);
    tile(k, tk, std::false_type{});
    wait_vmem();
    __syncthreads();
    tk = tk1;
  }
  for (; k < n_list; ++k) {
    const int tk1 = k + 1 < n_list ? tile_at(k + 1) : -1;
    if (tk1 >= 0) issue_tile(tk1 * kBC, (k & 1) ^ 1);
    if (tk == last) tile(k, tk, std::true_type{});
    wait_vmem();
    __syncthreads();
    tk = tk1;
  }

  // ---- epilogue: register r of tile dt holds head-dim element
  // dt*32 + 8*(r/4) + 4*h2 + r%4 of query qi
  if (qi < L) {
    uint16_t* dqp = a.dq + (int64_t)(start + qi) * ld + (int64_t)h * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = dt * 32 + 8 * g + 4 * h2;
        const u32x2 pk = {pack2<BF16>(qacc[dt][4 * g + 0] * a.scale, qacc[dt][4 * g + 1] * a.scale),
                          pack2<BF16>(qacc[dt][4 * g + 2] * a.scale, qacc[dt][4 * g + 3] * a.scale)};
        *reinterpret_cast<u32x2*>(dqp + d0) = pk;
      }
  }
}

// ---------------------------------------------------------------- dK, dV
// Software pipeline over 32-query halves of the 64-query tiles, one wave per
// SIMD: while the VALU turns S, dP of one half into Z and dS, the matrix cores
// already compute S, dP of the next half; then dV, dK take the first half's
// products.  Q/dO tiles are multi-buffered in LDS (kv_buffers: t in use,
// t + 1 read by the look-ahead products, later tiles landing).
//
// Geometry per head size.  Up to 192 a workgroup accumulates every column of
// dK and dV of its keys.  At 256 the accumulators (256 registers) and the K, V
// fragments (128) do not fit one wave, so the columns are split over
// kv_splits workgroups per key block: each recomputes S and dP over all of D
// and accumulates D / kv_splits columns.  The LDS holds four Q/dO tile
// buffers up to 128, three up to 192 (120-144 KB) and two at 256 (128 KB).
template <int D> constexpr int kv_splits() { return D > 192 ? 2 : 1; }
template <int D> constexpr int kv_cols() { return D / kv_splits<D>(); }
template <int D> constexpr int kv_buffers() { return D <= 128 ? 4 : (D <= 192 ? 3 : 2); }

template <int D, bool BF16>
struct KVState {
  u32x4 kf[D / 16], vf[D / 16];                // K, V fragments of this lane's key (all D)
  f32x16 dv[kv_cols<D>() / 32], dk[kv_cols<D>() / 32];  // the accumulated columns
};

// Per-lane LDS read addresses of one tile: operand reads (chunk pairs s even
// / odd) and transpose reads (rows +0 / +8) of the Q and dO tiles.  They are
// made opaque to the compiler so that every read of the tile becomes one of
// these registers plus an immediate offset.
struct TileAddr {
  uint32_t q0, q1, g0, g1;
};

__device__ __forceinline__ TileAddr tile_addr(uint32_t qb, uint32_t gb, uint32_t b0, uint32_t b1) {
  TileAddr t{qb + b0, qb + b1, gb + b0, gb + b1};
  asm volatile("" : "+v"(t.q0), "+v"(t.q1), "+v"(t.g0), "+v"(t.g1));
  return t;
}

// 32x32x16 product accumulated in place in VGPRs (inline assembly, so the
// result stays in VGPRs even where the compiler keeps its own products in
// AGPRs).  The compiler does not see these as matrix products: a VALU read
// of the result must come at least 19 wait states after the product
// (mfma_vgpr_wait), which the callers guarantee.
template <bool BF16>
__device__ __forceinline__ void mfma32_v(f32x16& acc, u32x4 a, u32x4 b) {
  if constexpr (BF16)
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
  else
    asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
template <bool BF16>
__device__ __forceinline__ void mfma32_v0(f32x16& acc, u32x4 a, u32x4 b) {
  if constexpr (BF16)
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
  else
    asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_vgpr_wait() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 4" ::: "memory"); }

// S = Q K^T and dP = dO V^T for queries 32qt .. 32qt+31 of a tile (pipeline
// prologue only; the loop computes them inside dkdv_half).
template <int D, bool BF16>
__device__ __forceinline__ void dkdv_sdp(const KVState<D, BF16>& st, const TileAddr& op, int qt, f32x16& sacc,
                                         f32x16& pacc) {
  using T = MTile<D, kBR>;
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    const uint32_t qa = (s & 1) ? op.q1 : op.q0, ga = (s & 1) ? op.g1 : op.g0;
    const u32x4 x = lds_read16_at(qa + T::opnd_off(qt, s)), y = lds_read16_at(ga + T::opnd_off(qt, s));
    if (s == 0) {
      mfma32_v0<BF16>(sacc, x, st.kf[s]);
      mfma32_v0<BF16>(pacc, y, st.vf[s]);
    } else {
      mfma32_v<BF16>(sacc, x, st.kf[s]);
      mfma32_v<BF16>(pacc, y, st.vf[s]);
    }
  }
  mfma_vgpr_wait();
}

// Where a 32-query half lives: its tile's LSE*log2(e) and D in LDS (offset
// by this lane half's first query), the tile's first query, and which half.
struct HalfCtx {
  uint32_t lb, db;
  int i0, qt;
  uint32_t kb;  // dropout: bit r set if element r is kept
};

// Value of lane 8*(l/8) + 7 - l%8 in lane l (DPP half-row mirror; every
// lane of the octet must be active).
__device__ __forceinline__ uint32_t octet_mirror(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xf, 0xf, false);
}

// Keep bits of this lane's key against the 64 queries of the tile at i0:
// bit 16*qt + r for element r of half qt (query i0 + 32qt + 8*(r/4) +
// 4*(lane/32) + r%4), i.e. bit 4*run + e for query i0 + 8*run + 4*(lane/32) + e.
// A Philox block (counter (q, kj/8, h, b)) holds the 16-bit values of one
// query against an aligned group of eight keys, which eight consecutive lanes
// own (lane mod 8 = kj mod 8).  Round g (0..3): lane c of an octet in lane
// half h2 hashes query i0 + 8*(2g + h2) + c, so every block is computed once;
// the octet gathers its 8 x 8 comparison bits with three DPP steps, the lane
// halves swap theirs, and each lane keeps the bits of its own key.

// Philox counter of round g.
__device__ __forceinline__ void keep_counter(int i0, int g, int h2, int kj, int h, int b, uint32_t (&c)[4]) {
  c[0] = (uint32_t)(i0 + 8 * (2 * g + h2) + (kj & 7));
  c[1] = (uint32_t)kj >> 3;
  c[2] = (uint32_t)h;
  c[3] = (uint32_t)b;
}

// Comparisons of a finished block: bit 8k + c of lo (keys 0..3 of the group)
// and of hi (keys 4..7, k - 4): query c of the run kept against key k.
__device__ __forceinline__ void keep_compare(const uint32_t (&r)[4], uint32_t t, int c, uint32_t& lo,
                                             uint32_t& hi) {
  lo = (keep16(r[0], 0, t) ? 1u : 0u) | (keep16(r[0], 1, t) ? 0x100u : 0u) |
       (keep16(r[1], 0, t) ? 0x10000u : 0u) | (keep16(r[1], 1, t) ? 0x1000000u : 0u);
  hi = (keep16(r[2], 0, t) ? 1u : 0u) | (keep16(r[2], 1, t) ? 0x100u : 0u) |
       (keep16(r[3], 0, t) ? 0x10000u : 0u) | (keep16(r[3], 1, t) ? 0x1000000u : 0u);
  lo <<= c;
  hi <<= c;
}

// The octet's 64 comparison bits in every lane of it.
__device__ __forceinline__ void keep_gather(uint32_t& lo, uint32_t& hi) {
  lo |= quad_perm<1, 0, 3, 2>(lo);
  hi |= quad_perm<1, 0, 3, 2>(hi);
  lo |= quad_perm<2, 3, 0, 1>(lo);
  hi |= quad_perm<2, 3, 0, 1>(hi);
  lo |= octet_mirror(lo);
  hi |= octet_mirror(hi);
}

// Tile bits 8g .. 8g+7 from the gathered comparisons of round g.
__device__ __forceinline__ uint32_t keep_extract(uint32_t lo, uint32_t hi, int c, int h2) {
  // bit q: query q of this half's run (2g + h2) kept against this lane's key
  uint32_t mine = ((c < 4 ? lo : hi) >> (8 * (c & 3))) & 0xFFu;
  uint32_t other = mine;
  permlane32_swap(mine, other);  // mine: run 2g (lanes 0-31), other: run 2g + 1 (lanes 32-63)
  const uint32_t sh = 4 * h2;
  return ((mine >> sh) & 0xFu) | (((other >> sh) & 0xFu) << 4);
}

// All of a tile's keep bits in one compact loop (the pipeline prologue).
__device__ __forceinline__ uint32_t dkdv_tile_keep(const BwdArgs& a, int b, int h, int i0, int h2, int kj) {
  uint32_t bits = 0;
#pragma unroll 1
  for (int g = 0; g < 4; ++g) {
    uint32_t r[4];
    keep_counter(i0, g, h2, kj, h, b, r);
#pragma unroll
    for (int k = 0; k < 10; ++k) philox_round(r, a.seed_lo, a.seed_hi, k);
    uint32_t lo, hi;
    keep_compare(r, a.drop_thresh, kj & 7, lo, hi);
    keep_gather(lo, hi);
    bits |= keep_extract(lo, hi, kj & 7, h2) << (8 * g);
  }
  return bits;
}

// The same bits in 32 slices, for a tile whose hashing is spread over the
// products of the tile before it (one slice per look-ahead product):
// slice 8g + p of round g runs Philox rounds 2p, 2p + 1 (p < 5), the
// comparisons (p = 5), the octet gather (p = 6) or the extraction (p = 7).
struct KeepTask {
  uint32_t c[4];
  uint32_t lo, hi, bits;
};

__device__ __forceinline__ void dkdv_keep_slice(const BwdArgs& a, int b, int h, int i0, int h2, int kj,
                                                KeepTask& k, int s) {
  const int g = s >> 3, p = s & 7;
  if (p == 0) {
    keep_counter(i0, g, h2, kj, h, b, k.c);
    if (g == 0) k.bits = 0;
  }
  if (p < 5) {
    philox_round(k.c, a.seed_lo, a.seed_hi, 2 * p);
    philox_round(k.c, a.seed_lo, a.seed_hi, 2 * p + 1);
  } else if (p == 5) {
    keep_compare(k.c, a.drop_thresh, kj & 7, k.lo, k.hi);
  } else if (p == 6) {
    keep_gather(k.lo, k.hi);
  } else {
    k.bits |= keep_extract(k.lo, k.hi, kj & 7, h2) << (8 * g);
  }
}

// P, Z and dS of element r of a half (register r of S, dP: query
// 32qt + 8*(r/4) + 4*(lane/32) + r%4 of this lane's key kj).
template <bool MASK, bool DROPOUT>
__device__ __forceinline__ void dkdv_elem(const BwdArgs& a, float s, float dp, float lse2, float dd, const HalfCtx& c,
                                          int r, int kj, int h2, float& z, float& ds) {
  const int qi = c.i0 + c.qt * 32 + 8 * (r >> 2) + 4 * h2 + (r & 3);
  float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s, a.scale_log2, -lse2));
  if (MASK && kj > qi) p = 0.f;
  z = p;
  if constexpr (DROPOUT) {
    const float kfac = (c.kb >> r) & 1u ? a.drop_rescale : 0.f;
    dp *= kfac;
    z = p * kfac;
  }
  ds = p * (dp - dd);
}

__device__ __forceinline__ f32x4 lds_f32x4(uint32_t addr) {
  return *(const __attribute__((address_space(3))) f32x4*)(uintptr_t)addr;
}

// One 32-query half h of the pipeline, in a fixed instruction order
// (sched_barrier fences keep the compiler from regrouping it).  On entry
// sacc, pacc hold S, dP of h and zpk/spk its packed Z, dS pairs 0..3
// (elements 0..7).
//   phase 1: the look-ahead products S, dP of the next half (operands of half
//            nqt of the tile at nop, read kPF products ahead), with elements
//            8..15 of h computed between them;
//   phase 2: dV += Z^T dO and dK += dS^T Q for h (transpose reads kPF2
//            products ahead), with elements 0..7 of the next half computed
//            between them once its S, dP are complete.
// Either phase then carries about three VALU instructions per product, few
// enough for the wave to issue them while its products run.  hook(i) runs
// after look-ahead product i (the caller issues its tile loads there, so that
// their issue overlaps the products).  On return sacc, pacc, zpk[0..3],
// spk[0..3] describe the next half.
template <int D, bool BF16, bool MASK, bool DROPOUT, bool PF_NEXT, typename Hook, typename Mid>
__device__ __forceinline__ void dkdv_half(const BwdArgs& a, KVState<D, BF16>& st, f32x16& sacc, f32x16& pacc,
                                          uint32_t (&zpk)[8], uint32_t (&spk)[8], u32x4 (&pf)[4],
                                          const TileAddr& nop, const TileAddr& nnop, int nnqt, const TileAddr& tr,
                                          const HalfCtx& cur, const HalfCtx& nxt, int kj, int h2,
                                          Hook&& hook, Mid&& mid) {
  using T = MTile<D, kBR>;
  constexpr int kNP = D / 8;  // look-ahead products (S and dP, D/16 k-steps each)
  // LDS operand reads in flight (products ahead); two at 256, where the
  // register file is full
  constexpr int kPF = (D >= 64 && D <= 192) ? 4 : 2;
  static_assert(kNP >= 2 * kPF, "prefetch window exceeds a phase");
  auto opnd = [&](const TileAddr& t, int qt, int i) {
    const int s = i >> 1;
    const uint32_t base = (i & 1) ? ((s & 1) ? t.g1 : t.g0) : ((s & 1) ? t.q1 : t.q0);
    return lds_read16_at(base + T::opnd_off(qt, s));
  };
  constexpr int kDT = kv_cols<D>() / 32;  // accumulated 32-column tiles (tr addresses start at the first)
  constexpr int kNA = 2 * 2 * kDT;         // dV, dK products
  auto tr_pair = [&](int j) {
    const int mm = j / (2 * kDT), dt = (j >> 1) % kDT;
    const uint32_t o = T::tr_off(2 * cur.qt + mm, dt);
    const uint32_t b0 = (j & 1) ? tr.q0 : tr.g0, b1 = (j & 1) ? tr.q1 : tr.g1;
    const u32x2 x0 = lds_read_tr_at(b0 + o), x1 = lds_read_tr_at(b1 + o);
    return u32x4{x0[0], x0[1], x1[0], x1[1]};
  };

  // ---- phase 1: look-ahead S, dP; elements 8..15 of h.  Operands 0..3
  // arrive in pf (read during the previous half); the last steps start the
  // transpose reads of phase 2.
  u32x4 ob[kNP];
  u32x4 tb[kNA];
#pragma unroll
  for (int i = 0; i < kPF; ++i) ob[i] = pf[i];
  const int qoff = cur.qt * 32;
  f32x4 l4a = lds_f32x4(cur.lb + 4 * (qoff + 16)), d4a = lds_f32x4(cur.db + 4 * (qoff + 16));
  f32x4 l4b = lds_f32x4(cur.lb + 4 * (qoff + 24)), d4b = lds_f32x4(cur.db + 4 * (qoff + 24));
  __builtin_amdgcn_sched_barrier(0);
  f32x16 ns, np;
  float zprev = 0.f, dsprev = 0.f;
#pragma unroll
  for (int i = 0; i < kNP; ++i) {
    const int s = i >> 1;
    if (i < 2) {
      if (i & 1)
        mfma32_v0<BF16>(np, ob[i], st.vf[s]);
      else
        mfma32_v0<BF16>(ns, ob[i], st.kf[s]);
    } else {
      if (i & 1)
        mfma32_v<BF16>(np, ob[i], st.vf[s]);
      else
        mfma32_v<BF16>(ns, ob[i], st.kf[s]);
    }
    if (i + kPF < kNP)
      ob[i + kPF] = opnd(nop, nxt.qt, i + kPF);
    else
      tb[i + kPF - kNP] = tr_pair(i + kPF - kNP);
    hook(i);  // work the caller spreads over the products (tile loads)
#pragma unroll
    for (int r = 8 + (i * 8) / kNP; r < 8 + ((i + 1) * 8) / kNP; ++r) {
      const f32x4& l4 = r < 12 ? l4a : l4b;
      const f32x4& d4 = r < 12 ? d4a : d4b;
      float z, ds;
      dkdv_elem<MASK, DROPOUT>(a, sacc[r], pacc[r], l4[r & 3], d4[r & 3], cur, r, kj, h2, z, ds);
      if (r & 1) {
        zpk[r >> 1] = pack2<BF16>(zprev, z);
        spk[r >> 1] = pack2<BF16>(dsprev, ds);
      } else {
        zprev = z;
        dsprev = ds;
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  const u32x4 zf[2] = {u32x4{zpk[0], zpk[1], zpk[2], zpk[3]}, u32x4{zpk[4], zpk[5], zpk[6], zpk[7]}};
  const u32x4 sf[2] = {u32x4{spk[0], spk[1], spk[2], spk[3]}, u32x4{spk[4], spk[5], spk[6], spk[7]}};
  mid();  // the caller's work between the phases (it may complete nxt)

  // ---- phase 2: product j = (slice mm, head-dim tile dt, dV or dK) of h;
  // elements 0..7 of the next half, starting once ns, np are complete; the
  // last steps read the first operands of the next half's look-ahead
  // products (half nnqt of the tile at nnop) into pf.
  constexpr int kLag = 2;  // products to wait before reading ns, np
  static_assert(kNA >= 2 * kPF, "prefetch window exceeds a phase");
  const int noff = nxt.qt * 32;
  f32x4 l4c = lds_f32x4(nxt.lb + 4 * noff), d4c = lds_f32x4(nxt.db + 4 * noff);
  f32x4 l4d = lds_f32x4(nxt.lb + 4 * (noff + 8)), d4d = lds_f32x4(nxt.db + 4 * (noff + 8));
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < kNA; ++j) {
    const int mm = j / (2 * kDT), dt = (j >> 1) % kDT;
    if (j & 1)
      st.dk[dt] = mfma32<BF16>(sf[mm], tb[j], st.dk[dt]);
    else
      st.dv[dt] = mfma32<BF16>(zf[mm], tb[j], st.dv[dt]);
    if (j == 0) mfma_vgpr_wait();  // ns, np (read from j = kLag on) are complete
    if (j + kPF < kNA)
      tb[j + kPF] = tr_pair(j + kPF);
    else if (PF_NEXT)  // (otherwise the caller reads them once they have landed)
      pf[j + kPF - kNA] = opnd(nnop, nnqt, j + kPF - kNA);
    if (j >= kLag) {
      constexpr int kSpan = kNA - kLag;
#pragma unroll
      for (int r = ((j - kLag) * 8) / kSpan; r < ((j - kLag + 1) * 8) / kSpan; ++r) {
        const f32x4& l4 = r < 4 ? l4c : l4d;
        const f32x4& d4 = r < 4 ? d4c : d4d;
        float z, ds;
        dkdv_elem<MASK, DROPOUT>(a, ns[r], np[r], l4[r & 3], d4[r & 3], nxt, r, kj, h2, z, ds);
        if (r & 1) {
          zpk[r >> 1] = pack2<BF16>(zprev, z);
          spk[r >> 1] = pack2<BF16>(dsprev, ds);
        } else {
          zprev = z;
          dsprev = ds;
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  sacc = ns;
  pacc = np;
}

template <int D, bool BF16, bool CAUSAL, bool DROPOUT, bool SPARSE, bool KB = false>
__global__ __launch_bounds__(kThreads, 1) void fa_bwd_dkdv_kernel(BwdArgs a) {
  static_assert(!KB || (DROPOUT && !SPARSE), "keep bits: dense dropout instantiations only");
  static_assert(!KB || (kBR == 64 && kBKV == 128), "keep-bit tiles: 64 queries by two 64-key words pairs");
  using T = MTile<D, kBR>;
  constexpr int kNB = kv_buffers<D>();  // Q/dO/LSE/D tile buffers
  constexpr int kAhead = kNB - 1;       // tiles loaded ahead of the one in use
  constexpr int kDA = kv_cols<D>();     // dK, dV columns this workgroup accumulates
  __shared__ __attribute__((aligned(1024))) uint16_t qs[kNB][T::kElems];
  __shared__ __attribute__((aligned(1024))) uint16_t gs[kNB][T::kElems];
  __shared__ __attribute__((aligned(16))) float ls[kNB][kBR];
  __shared__ __attribute__((aligned(16))) float dls[kNB][kBR];
  __shared__ __attribute__((aligned(16))) float spare[64];
  // keep bits: the stored words of a tile's 64 queries against the block's
  // 128 keys, four planes of 64 rows (plane p: key tile 2*kb + p/2, key
  // half p%2 -- the 32 keys of wave p)
  __shared__ __attribute__((aligned(1024))) uint32_t kbs[KB ? kNB : 1][KB ? 256 : 4];
  // block-sparse: the query tiles the workgroup visits, in order
  __shared__ uint16_t tlist[SPARSE ? kMaxSparseTiles : 1];
  __shared__ uint8_t tflag[SPARSE ? kMaxSparseTiles : 1];
  __shared__ int tcount[1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h2 = lane >> 5;
  const int l32 = lane & 31;

  // Workgroup -> (b, h, key block, column split): the key blocks of one
  // head share an XCD, two heads at a time where B*H allows, key blocks first
  // to last (causal: the first see the most queries).  The key blocks of a
  // head start their causal query sweeps at different tiles, so with all of
  // an XCD's heads at once its L2 could not hold their Q and dO tiles: at
  // B 4, H 8, N 4096, d 128 causal this order fetches 151 MB instead of
  // about 470 MB in the same time (one head at a time: 143 MB, 3% slower).
  const int BH = a.B * a.H;
  int bh, rest;
  xcd_head_order<kKvHeadGroup>(blockIdx.x, BH, a.nkb * kv_splits<D>(), bh, rest);
  const int kb = rest / kv_splits<D>();
  const int split = rest % kv_splits<D>();
  const int c0 = split * kDA;  // first accumulated column
  const int b = bh / a.H;
  const int h = bh % a.H;
  int start, L;
  seq_range(a, b, start, L);
  const int j0 = kb * kBKV;
  if (j0 >= L) return;

  const int64_t ld = a.ld;
  const int64_t hd = (int64_t)a.H * D;
  const uint32_t row_bytes = (uint32_t)ld * 2;
  const uint32_t grow_bytes = (uint32_t)hd * 2;
  const int kw0 = j0 + 32 * w;  // first key of this wave
  const int kj = kw0 + l32;     // key owned by this lane

  KVState<D, BF16> st;
  {
    // keys past the end read as zeros
    const int rows = max(0, min(32, L - kw0));
    const int64_t tok = start + min(kw0, L - 1);
    const uint32_t bytes = rows > 0 ? (uint32_t)(rows - 1) * row_bytes + D * 2 : 0u;
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(a.k + tok * ld + (int64_t)h * D, bytes);
    const __amdgpu_buffer_rsrc_t vr = make_rsrc(a.v + tok * ld + (int64_t)h * D, bytes);
    const uint32_t off = (uint32_t)l32 * row_bytes + 16 * h2;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      st.kf[s] = buffer_load16(kr, off + 32 * s);
      st.vf[s] = buffer_load16(vr, off + 32 * s);
    }
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      asm volatile("" : "+v"(st.kf[s]));
      asm volatile("" : "+v"(st.vf[s]));
    }
#pragma unroll
    for (int dt = 0; dt < kDA / 32; ++dt) {
      st.dv[dt] = f32x16{};
      st.dk[dt] = f32x16{};
      // the accumulators live in AGPRs for the whole loop (only the matrix
      // cores touch them until the epilogue)
      asm volatile("" : "+a"(st.dv[dt]));
      asm volatile("" : "+a"(st.dk[dt]));
    }
  }

  // Query tiles that can see the keys: all, or (causal) from the tile holding
  // query j0 on.  Rows past the end of the sequence load as zeros (Q = dO = 0,
  // LSE = D = 0), which gives P = 1, dP = 0 and dS = 0: no contribution.
  const int i_begin = CAUSAL ? (j0 / kBR) * kBR : 0;
  const int ntiles = (L - i_begin + kBR - 1) / kBR;
  const uint16_t* qbase = a.q + (int64_t)start * ld + (int64_t)h * D;
  const uint16_t* gbase = a.dout + (int64_t)start * hd + (int64_t)h * D;
  const float* lbase = a.lse2 + (int64_t)start * a.H + h;
  const float* dbase = a.delta + (int64_t)start * a.H + h;
  const uint32_t qs0 = lds_addr(qs), gs0 = lds_addr(gs), ls0 = lds_addr(ls), dls0 = lds_addr(dls);
  const uint32_t hstride4 = (uint32_t)a.H * 4;  // bytes between consecutive tokens of LSE and D

  // the stored keep words of this head (at most 512 MB: N <= 65536); lane l
  // of the tile's 1 KB load takes rows 4*(l%16) .. +3 of plane l/16
  const __amdgpu_buffer_rsrc_t kbr =
      KB ? make_rsrc(a.kbits + (int64_t)bh * a.nkt * 2 * a.kbn, (uint32_t)((uint64_t)a.nkt * 2 * a.kbn * 4))
         : make_rsrc(nullptr, 0u);
  auto kbits_off = [&](int il) __attribute__((always_inline)) -> uint32_t {
    if (il < 0) return 0xFFFFFFF0u;  // absent tile: out of range, the load fills zeros
    const uint32_t p = (uint32_t)lane >> 4;
    const uint32_t word = ((uint32_t)(j0 / 64 + (int)(p >> 1)) * 2 + (p & 1)) * (uint32_t)a.kbn + (uint32_t)il +
                          4 * ((uint32_t)lane & 15);
    return word * 4;
  };
  auto issue_tile = [&](int i0, int buf) {
    const int rows = min(kBR, L - i0);
    if constexpr (KB)
      if (w == 2) buffer_load_lds16_addr(kbr, lds_addr(kbs[buf]), kbits_off(i0));
    const __amdgpu_buffer_rsrc_t qr = make_rsrc(qbase + (int64_t)i0 * ld, (uint32_t)(rows - 1) * row_bytes + D * 2);
    const __amdgpu_buffer_rsrc_t gr = make_rsrc(gbase + (int64_t)i0 * hd, (uint32_t)(rows - 1) * grow_bytes + D * 2);
    static_assert(T::kBlocks % kWaves == 0, "tile blocks must split evenly over the waves");
#pragma unroll
    for (int u = 0; u < T::kBlocks / kWaves; ++u) {
      T::load(qr, qs0 + buf * T::kBytes, row_bytes, u * kWaves + w, lane);
      T::load(gr, gs0 + buf * T::kBytes, grow_bytes, u * kWaves + w, lane);
    }
    if (w == 0) {
      const __amdgpu_buffer_rsrc_t lr = make_rsrc(lbase + (int64_t)i0 * a.H, (uint32_t)(rows - 1) * a.H * 4 + 4);
      buffer_load_lds4(lr, ls[buf], (uint32_t)lane * a.H * 4);
    } else if (w == 1) {
      const __amdgpu_buffer_rsrc_t dr = make_rsrc(dbase + (int64_t)i0 * a.H, (uint32_t)(rows - 1) * a.H * 4 + 4);
      buffer_load_lds4(dr, dls[buf], (uint32_t)lane * a.H * 4);
    }
  };

  const uint32_t ob0 = T::opnd_base(lane, 0), ob1 = T::opnd_base(lane, 1);
  // transpose reads (dV, dK products) start at the first accumulated column:
  // 32 columns are 2 KB of a tile
  const uint32_t tb0 = T::tr_base(lane, 0) + 64 * c0, tb1 = T::tr_base(lane, 1) + 64 * c0;

  // Visited query tiles: all tiles 0 .. ntiles-1 (from i_begin), or
  // (block-sparse) the listed ones.  Buffers follow the position k in that
  // sequence; tile_at(k) is the tile index.
  int n_list = ntiles;
  if constexpr (SPARSE) {
    if (w == 0) {
      const uint8_t* mcol = a.bmask + ((int64_t)b * a.H + h) * a.nb * a.nb + j0 / kMaskBlock;
      const int n = build_tile_list(mcol, nullptr, i_begin / kBR, a.nb, ntiles, tlist, tflag, lane);
      if (lane == 0) tcount[0] = n;
    }
    __syncthreads();
    n_list = __builtin_amdgcn_readfirstlane(tcount[0]);
  }
  auto tile_at = [&](int k) __attribute__((always_inline)) -> int {
    if constexpr (SPARSE) return __builtin_amdgcn_readfirstlane(tlist[k]);
    else return k;
  };
  const int t_first = n_list > 0 ? tile_at(0) : 0;

  // Loads of visited tile tkl (-1: none) into buffer lbuf, as one wave's
  // share: part k < 2 * kNU is a Q (even) or dO (odd) block, part 2 * kNU
  // the LSE (wave 0) or D (wave 1) row; waves 2 and 3 send an empty load to
  // a spare row, so every wave issues kTileLoads loads per tile.  An absent
  // tile has empty buffer ranges: its loads fetch nothing and fill the
  // buffer with zeros.
  constexpr int kNU = T::kBlocks / kWaves;  // blocks per tensor per wave
  constexpr int kTileLoads = 2 * kNU + 1;
  struct TileLoads {
    __amdgpu_buffer_rsrc_t qr, gr, xr;
    uint32_t qdst, gdst, xdst;
    uint32_t bdst, boff;  // keep bits (wave 2 loads them instead of its empty load)
  };
  const uint32_t xoff = (uint32_t)lane * hstride4;
  auto tile_loads = [&](int tkl, int lbuf) __attribute__((always_inline)) {
    const int il = i_begin + max(tkl, 0) * kBR;
    const int rows = tkl >= 0 ? min(kBR, L - il) : 0;
    const int64_t tok = min(il, L - 1);
    TileLoads x;
    x.qr = make_rsrc(qbase + tok * ld, rows > 0 ? (uint32_t)(rows - 1) * row_bytes + D * 2 : 0u);
    x.gr = make_rsrc(gbase + tok * hd, rows > 0 ? (uint32_t)(rows - 1) * grow_bytes + D * 2 : 0u);
    x.xr = w < 2 ? make_rsrc((w == 0 ? lbase : dbase) + tok * a.H, rows > 0 ? (uint32_t)(rows - 1) * a.H * 4 + 4 : 0u)
                 : make_rsrc(nullptr, 0u);
    x.qdst = qs0 + lbuf * T::kBytes;
    x.gdst = gs0 + lbuf * T::kBytes;
    x.xdst = w == 0 ? ls0 + lbuf * kBR * 4 : w == 1 ? dls0 + lbuf * kBR * 4 : lds_addr(spare);
    if constexpr (KB) {
      x.bdst = lds_addr(kbs[lbuf]);
      x.boff = kbits_off(tkl >= 0 ? il : -1);
    }
    return x;
  };
  auto tile_load_part = [&](const TileLoads& x, int k) __attribute__((always_inline)) {
    if (KB && k == 2 * kNU && w == 2)
      buffer_load_lds16_addr(kbr, x.bdst, x.boff);
    else if (k == 2 * kNU)
      buffer_load_lds4_addr(x.xr, x.xdst, xoff);
    else if (k & 1)
      T::load(x.gr, x.gdst, grow_bytes, (k >> 1) * kWaves + w, lane);
    else
      T::load(x.qr, x.qdst, row_bytes, (k >> 1) * kWaves + w, lane);
  };

  // prologue loads: tiles 0 and (with two or more tiles ahead) 1 landed,
  // tiles 2 .. kAhead - 1 in flight
  if (n_list > 0) issue_tile(i_begin + t_first * kBR, 0);
  if (kAhead >= 2 && n_list > 1) issue_tile(i_begin + tile_at(1) * kBR, 1);
  wait_vmem();
  __syncthreads();
  if constexpr (kAhead >= 3) {
    static_assert(kAhead == 3, "at most three tiles ahead");
    const TileLoads x = tile_loads(n_list > 2 ? tile_at(2) : -1, 2);
#pragma unroll
    for (int k = 0; k <= 2 * kNU; ++k) tile_load_part(x, k);
  }

  // pipeline prologue: S, dP and elements 0..7 of the first half, and the
  // first operands of its look-ahead products (half 1 of tile 0)
  // dropout keep bits of the tile in use (bit 16*half + element)
  // keep bits: runs of four queries 8*run + 4*h2 + e of the tile in buffer
  // buf against this lane's key (bit l32 of the row words of plane w), at
  // bits e of the result
  auto kb_run = [&](int buf, int run) __attribute__((always_inline)) -> uint32_t {
    const u32x4 wd = *(const __attribute__((address_space(3))) u32x4*)(uintptr_t)(
        lds_addr(kbs[buf]) + 4 * (64 * w + 8 * run + 4 * h2));
    return ((wd[0] >> l32) & 1u) | (((wd[1] >> l32) & 1u) << 1) | (((wd[2] >> l32) & 1u) << 2) |
           (((wd[3] >> l32) & 1u) << 3);
  };
  uint32_t kb_cur = 0;
  if constexpr (KB) {
#pragma unroll
    for (int run = 0; run < 8; ++run) kb_cur |= kb_run(0, run) << (4 * run);
  } else if constexpr (DROPOUT) {
    kb_cur = dkdv_tile_keep(a, b, h, i_begin + t_first * kBR, h2, kj);
  }
  f32x16 sacc, pacc;
  uint32_t zpk[8], spk[8];
  u32x4 pf[4];
  const TileAddr op0 = tile_addr(qs0, gs0, ob0, ob1);
  dkdv_sdp<D, BF16>(st, op0, 0, sacc, pacc);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int s = i >> 1;
    const uint32_t base = (i & 1) ? ((s & 1) ? op0.g1 : op0.g0) : ((s & 1) ? op0.q1 : op0.q0);
    pf[i] = lds_read16_at(base + T::opnd_off(1, s));
  }
  {
    const HalfCtx c0{ls0 + 16 * h2, dls0 + 16 * h2, i_begin + t_first * kBR, 0, kb_cur & 0xffffu};
    float zprev = 0.f, dsprev = 0.f;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const f32x4 l4 = lds_f32x4(c0.lb + 4 * 8 * (r >> 2)), d4 = lds_f32x4(c0.db + 4 * 8 * (r >> 2));
      float z, ds;
      dkdv_elem<CAUSAL, DROPOUT>(a, sacc[r], pacc[r], l4[r & 3], d4[r & 3], c0, r, kj, h2, z, ds);
      if (r & 1) {
        zpk[r >> 1] = pack2<BF16>(zprev, z);
        spk[r >> 1] = pack2<BF16>(dsprev, ds);
      } else {
        zprev = z;
        dsprev = ds;
      }
    }
  }

  // Iteration at position t of the visited tiles (tiles tk, tk1, tka at
  // positions t, t+1, t+kAhead; -1 past the end).
  auto iteration = [&](int t, int tk, int tk1, int tka, auto mask) {
    constexpr bool kMask = decltype(mask)::value;
    const int buf = t % kNB;
    const int nbuf = (t + 1) % kNB;
    const int i0 = i_begin + tk * kBR;
    // With two or more tiles ahead, tile t + 1 has landed here (loads
    // complete in order: only tiles t + 2 .. t + kAhead - 1 may still be in
    // flight).  Every wave is done with tile t - 1's buffers (the reads still
    // in flight here touch tiles t and t + 1 only).
    if constexpr (kAhead >= 2) wait_vmem_n<(kAhead - 2) * kTileLoads>();
    barrier_keep_lds_reads();

    // Loads of tile t + kAhead into buffer (t + kAhead) % kNB (tile t - 1's),
    // spread over the first half's look-ahead products: Q and dO blocks at
    // even products, LSE or D at product 1.
    const TileLoads x = tile_loads(tka, (t + kAhead) % kNB);
    static_assert(4 * kNU - 2 < D / 8, "the look-ahead products must carry every tile load");
    // Dropout: the next tile's keep bits, hashed in 32 slices spread over
    // the look-ahead products of both halves (where the VALU has room next
    // to the matrix cores); the second half's phase 2 reads them through n0.
    KeepTask kt;
    if constexpr (KB) kt.bits = 0;
    const int next_i0 = i_begin + max(tk1, 0) * kBR;
    auto keep_hook = [&](int half, int i) __attribute__((always_inline)) {
      if constexpr (KB) {
        // the next tile's stored bits (landed: loaded kAhead tiles ahead, or,
        // one ahead, waited for between the halves), read in the second half
        constexpr int kRuns = (8 + D / 8 - 1) / (D / 8);  // runs per look-ahead product
        if (half == 1)
#pragma unroll
          for (int run = i * kRuns; run < (i + 1) * kRuns && run < 8; ++run)
            kt.bits |= kb_run(nbuf, run) << (4 * run);
      } else if constexpr (DROPOUT) {
        constexpr int kPer = (32 + 2 * (D / 8) - 1) / (2 * (D / 8));  // slices per look-ahead product
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
          const int sl = (half * (D / 8) + i) * kPer + u;
          if (sl < 32) dkdv_keep_slice(a, b, h, next_i0, h2, kj, kt, sl);
        }
      }
    };
    auto load_hook = [&](int i) __attribute__((always_inline)) {
      if (i % 2 == 0 && i / 2 < 2 * kNU) tile_load_part(x, i / 2);
      if (i == 1) tile_load_part(x, 2 * kNU);
      keep_hook(0, i);
    };
    auto second_hook = [&](int i) __attribute__((always_inline)) { keep_hook(1, i); };

    const uint32_t qb = qs0 + buf * T::kBytes, gb = gs0 + buf * T::kBytes;
    const uint32_t nqb = qs0 + nbuf * T::kBytes, ngb = gs0 + nbuf * T::kBytes;
    const TileAddr op = tile_addr(qb, gb, ob0, ob1), tr = tile_addr(qb, gb, tb0, tb1);
    const TileAddr nop = tile_addr(nqb, ngb, ob0, ob1);
    uint32_t lb = ls0 + buf * kBR * 4 + 16 * h2, db = dls0 + buf * kBR * 4 + 16 * h2;
    uint32_t nlb = ls0 + nbuf * kBR * 4 + 16 * h2, ndb = dls0 + nbuf * kBR * 4 + 16 * h2;
    asm volatile("" : "+v"(lb), "+v"(db), "+v"(nlb), "+v"(ndb));
    const HalfCtx h0{lb, db, i0, 0, kb_cur & 0xffffu}, h1{lb, db, i0, 1, kb_cur >> 16};
    // first half of the next tile, whose keep bits the hooks finish before
    // the second half's phase 2 reads them
    HalfCtx n0{nlb, ndb, next_i0, 0, 0u};
    // On the last tile the look-ahead work reads a stale buffer and is
    // discarded; doing it anyway keeps the tile one basic block.  Masked
    // tiles come first, so the look-ahead into the next tile may use this
    // tile's masking.
    dkdv_half<D, BF16, kMask, DROPOUT, (kAhead >= 2)>(a, st, sacc, pacc, zpk, spk, pf, op, nop, 0, tr, h0, h1, kj,
                                                      h2, load_hook, []() {});
    if constexpr (DROPOUT) {
      // every slice ran in the first half and the second half's phase 1
      static_assert(2 * (D / 8) * ((32 + 2 * (D / 8) - 1) / (2 * (D / 8))) >= 32, "keep slices do not fit");
    }
    if constexpr (kAhead == 1) {
      // one tile ahead: tile t + 1 was issued at the start of this iteration;
      // wait for every wave's share before reading the first operands of its
      // look-ahead products (which the first half leaves to this point)
      wait_vmem();
      barrier_keep_lds_reads();
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int s = i >> 1;
        const uint32_t base = (i & 1) ? ((s & 1) ? nop.g1 : nop.g0) : ((s & 1) ? nop.q1 : nop.q0);
        pf[i] = lds_read16_at(base + T::opnd_off(0, s));
      }
    }
    dkdv_half<D, BF16, kMask, DROPOUT, true>(a, st, sacc, pacc, zpk, spk, pf, nop, nop, 1, tr, h1, n0, kj, h2,
                                             second_hook, [&]() __attribute__((always_inline)) {
                                               if constexpr (DROPOUT) n0.kb = kt.bits & 0xffffu;
                                             });
    if constexpr (DROPOUT) kb_cur = kt.bits;
  };
  // Causal: only the first two tiles (queries j0 .. j0+127) hold queries
  // before some key of the block, so only they are masked.
  int t = 0;
  int tk = n_list > 0 ? t_first : -1;
  int tk1 = n_list > 1 ? tile_at(1) : -1;
  auto tile_or_none = [&](int k) __attribute__((always_inline)) { return k < n_list ? tile_at(k) : -1; };
  if (CAUSAL)
    for (; t < n_list && tk < 2; ++t) {
      iteration(t, tk, tk1, tile_or_none(t + kAhead), std::true_type{});
      tk = tk1;
      tk1 = tile_or_none(t + 2);
    }
  for (; t < n_list; ++t) {
    iteration(t, tk, tk1, tile_or_none(t + kAhead), std::false_type{});
    tk = tk1;
    tk1 = tile_or_none(t + 2);
  }

#pragma unroll
  for (int dt = 0; dt < kDA / 32; ++dt) {
    asm volatile("" : "+a"(st.dv[dt]));
    asm volatile("" : "+a"(st.dk[dt]));
  }

  // ---- epilogue: dK = scale * dK, dV, staged through LDS as [key][d] rows
  // (register r of tile dt: key 8*(r/4) + 4*h2 + r%4 of the wave, element
  // dt*32 + l32), then written back 16 bytes per lane.  The (empty) loads
  // of the last iterations still write the tile buffers: wait for them.
  wait_vmem();
  __syncthreads();
  constexpr int kRowE = kDA + 8;  // padded LDS row, 16-bit elements
  uint16_t* stage_k = qs[0];    // 128 rows x kRowE elements fit in each set of tile buffers
  uint16_t* stage_v = gs[0];
  static_assert(kBKV * kRowE <= kNB * T::kElems, "epilogue staging does not fit");
#pragma unroll
  for (int dt = 0; dt < kDA / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 32 * w + 8 * (r >> 2) + 4 * h2 + (r & 3);
      const uint32_t pk = pack2<BF16>(st.dk[dt][r] * a.scale, st.dv[dt][r]);
      stage_k[row * kRowE + dt * 32 + l32] = (uint16_t)(pk & 0xffff);
      stage_v[row * kRowE + dt * 32 + l32] = (uint16_t)(pk >> 16);
    }
  __syncthreads();
  constexpr int kCPR = kDA / 8;  // 16-byte chunks of the accumulated columns of a row
#pragma unroll
  for (int u = 0; u < kBKV * kCPR / kThreads; ++u) {
    const int c = tid + kThreads * u;
    const int row = c / kCPR;
    const int col = (c % kCPR) * 8;
    const int j = j0 + row;
    if (j < L) {
      const int64_t off = (int64_t)(start + j) * ld + (int64_t)h * D + c0 + col;
      *reinterpret_cast<u32x4*>(a.dk + off) = *reinterpret_cast<const u32x4*>(&stage_k[row * kRowE + col]);
      *reinterpret_cast<u32x4*>(a.dv + off) = *reinterpret_cast<const u32x4*>(&stage_v[row * kRowE + col]);
    }
  }
}

template <int D, bool BF16, bool CAUSAL, bool DROPOUT, bool SPARSE>
hipError_t launch_bwd_s(const AttnShape& s, BwdArgs args, int stages, hipStream_t stream) {
  args.nqb = (s.N + dq_rows<SPARSE, D>() - 1) / dq_rows<SPARSE, D>();
  // keep-bit instances: dense dropout with stored decisions
  constexpr bool kKB = DROPOUT && !SPARSE;
  const bool kb = kKB && args.kbits != nullptr;
  if (stages & kBwdDq) {
    const int64_t nb = (int64_t)args.nqb * s.B * s.H;
    if (nb > 0x7fffffff) return hipErrorInvalidConfiguration;
    if (kb)
      hipLaunchKernelGGL((fa_bwd_dq_kernel<D, BF16, CAUSAL, DROPOUT, SPARSE, kKB>), dim3((unsigned)nb),
                         dim3(64 * dq_waves<SPARSE, D>()), 0, stream, args);
    else
      hipLaunchKernelGGL((fa_bwd_dq_kernel<D, BF16, CAUSAL, DROPOUT, SPARSE>), dim3((unsigned)nb),
                         dim3(64 * dq_waves<SPARSE, D>()), 0, stream, args);
  }
  if (stages & kBwdKV) {
    const int64_t nb = (int64_t)args.nkb * s.B * s.H * kv_splits<D>();
    if (nb > 0x7fffffff) return hipErrorInvalidConfiguration;
    if (kb)
      hipLaunchKernelGGL((fa_bwd_dkdv_kernel<D, BF16, CAUSAL, DROPOUT, SPARSE, kKB>), dim3((unsigned)nb),
                         dim3(kThreads), 0, stream, args);
    else
      hipLaunchKernelGGL((fa_bwd_dkdv_kernel<D, BF16, CAUSAL, DROPOUT, SPARSE>), dim3((unsigned)nb),
                         dim3(kThreads), 0, stream, args);
  }
  return hipGetLastError();
}

template <int D, bool BF16, bool CAUSAL, bool DROPOUT>
hipError_t launch_bwd_t(const AttnShape& s, const BwdArgs& args, int stages, hipStream_t stream) {
  static_assert(D % 32 == 0 && D >= 32 && D <= 256, "head sizes: multiples of 32 up to 256");
  return args.bmask ? launch_bwd_s<D, BF16, CAUSAL, DROPOUT, true>(s, args, stages, stream)
                    : launch_bwd_s<D, BF16, CAUSAL, DROPOUT, false>(s, args, stages, stream);
}

template <int D, bool BF16>
hipError_t launch_bwd_d(const AttnShape& s, const BwdArgs& args, int stages, hipStream_t stream) {
  if (s.causal)
    return s.dropout ? launch_bwd_t<D, BF16, true, true>(s, args, stages, stream)
                     : launch_bwd_t<D, BF16, true, false>(s, args, stages, stream);
  return s.dropout ? launch_bwd_t<D, BF16, false, true>(s, args, stages, stream)
                   : launch_bwd_t<D, BF16, false, false>(s, args, stages, stream);
}

}  // namespace

hipError_t launch_backward(const AttnShape& s, const void* q, const void* k, const void* v, const void* o,
                           const float* lse, const void* dout, void* dq, void* dk, void* dv, float* delta,
                           float* lse2, int stages, hipStream_t stream) {
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
  a.delta = delta;
  a.lse2 = lse2;
  a.cu = s.cu;
  a.ld = s.ld;
  a.B = s.B;
  a.H = s.H;
  a.N = s.N;
  a.nqb = 0;  // set by the launcher from the workgroup size of the instance
  a.nkb = (s.N + kBKV - 1) / kBKV;
  a.kbits = s.dropout && !s.bmask ? s.keep_bits : nullptr;
  a.nkt = (s.N + 63) / 64;
  a.kbn = keep_bits_rows(s.N);
  a.scale = s.scale;
  a.scale_log2 = s.scale * kLog2e;
  a.drop_thresh = s.drop_thresh;
  a.drop_rescale = s.drop_rescale;
  a.seed_lo = (uint32_t)s.seed;
  a.seed_hi = (uint32_t)(s.seed >> 32);
  a.bmask = s.bmask;
  a.nb = s.nb;
  switch (s.d) {
    case 32: return s.bf16 ? launch_bwd_d<32, true>(s, a, stages, stream) : launch_bwd_d<32, false>(s, a, stages, stream);
    case 64: return s.bf16 ? launch_bwd_d<64, true>(s, a, stages, stream) : launch_bwd_d<64, false>(s, a, stages, stream);
    case 96: return s.bf16 ? launch_bwd_d<96, true>(s, a, stages, stream) : launch_bwd_d<96, false>(s, a, stages, stream);
    case 128: return s.bf16 ? launch_bwd_d<128, true>(s, a, stages, stream)
                            : launch_bwd_d<128, false>(s, a, stages, stream);
    case 160: return s.bf16 ? launch_bwd_d<160, true>(s, a, stages, stream)
                            : launch_bwd_d<160, false>(s, a, stages, stream);
    case 192: return s.bf16 ? launch_bwd_d<192, true>(s, a, stages, stream)
                            : launch_bwd_d<192, false>(s, a, stages, stream);
    default: return s.bf16 ? launch_bwd_d<256, true>(s, a, stages, stream)
                           : launch_bwd_d<256, false>(s, a, stages, stream);
  }
}

}  // namespace fa
