// Fused exact attention forward for gfx950 (MI355X).
//
// One workgroup = one (batch-or-sequence b, head h, block of kBR queries);
// eight waves (two per SIMD, so one wave's softmax overlaps the other's
// matrix products), each owning 32 consecutive queries.  The block-sparse
// instantiation uses four waves (128 queries, one mask row) and two
// workgroups per CU instead.  The kernel walks the
// key blocks the block needs (all of them, or only those left of the
// diagonal when causal), which is the tiling of the lab write-up
// "FlashAttention" (dpshk.com), section 3.1, with QK^T, softmax and PV fused
// as in the tiemojia.cn article's "kernel fusion" paragraph:
//   - K and V tiles (kBC keys) go straight from HBM to LDS (direct buffer
//     loads), double buffered: the next tile's loads are in flight while the
//     current tile is consumed.  The tiles use the MFMA-native LDS layout of
//     MTile, so operand and transpose reads are conflict-free and each is a
//     base register plus an immediate offset; LDS operands are read a few
//     products ahead of the product that consumes them.
//   - The wave computes S^T = K Q^T with v_mfma_f32_32x32x16 (Q stays in
//     registers as the B operand).  In that orientation each lane owns one
//     query and 16 keys per 32x32 tile, so the row max and row sum are
//     in-lane reductions plus one v_permlane32_swap.
//   - Online softmax (section 3.2 of the write-up): running max m and sum l
//     per query in fp32; the partial output is rescaled by e^{m_old - m_new};
//     exponentials use exp2 with scale*log2(e) folded in.
//   - O^T += V^T P^T: the P accumulator registers are already laid out as
//     the B operand (the key order inside each 16-key MFMA slice is
//     permuted, and V is read with the same permutation), V^T comes from the
//     LDS transpose read ds_read_b64_tr_b16.
//   - Epilogue: O = O / l in fp32, rounded once to bf16/fp16; LSE = m + ln l.
#include <type_traits>

#include "fa_device.hpp"
#include "fa_internal.h"

namespace fa {
namespace {

// Dense, heads up to 128: eight waves (two per SIMD, ping-pong), 256 queries
// share each K/V tile.  Block-sparse: four waves (one 128-query mask row per
// workgroup, so the tile list is exact), no ping-pong, two workgroups per CU
// for heads up to 128.  Heads above 128: four waves, one per SIMD and one
// workgroup per CU, so that each wave has the whole register file for its
// larger output tile (and the K/V double buffers of up to 128 KB fit in LDS).
template <bool SPARSE, int D> constexpr int waves() { return (SPARSE || D > 128) ? 4 : 8; }
template <bool SPARSE, int D> constexpr int rows_per_wg() { return 32 * waves<SPARSE, D>(); }
template <bool SPARSE, int D> constexpr int wgs_per_cu() { return (SPARSE && D <= 128) ? 2 : 1; }
constexpr int kBC = 64;           // keys per tile
// The partial output is rescaled only when a row max grows by more than this
// many powers of two; otherwise the stale max stays the reference, so the
// unnormalised probabilities stay below 2^8 (exact: O and l share the same
// reference, and O / l is taken once at the end).
constexpr float kRescaleLog2 = 8.0f;

struct FwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  const int32_t* cu;
  int64_t ld;
  int B, H, N, nqb;
  float scale_log2;
  uint32_t drop_thresh;
  float drop_rescale;
  uint32_t seed_lo, seed_hi;
  const uint8_t* bmask;  // block-sparse instantiations only: [B, H, nb, nb]
  int nb;
  uint32_t* kbits;  // keep-bit instantiations only: the decisions drawn (layout: fa_internal.h)
  int nkt;          // ceil(N / 64)
  int kbn;          // row stride of the keep-bit planes (N rounded up to 4)
};

template <int D, bool BF16, bool CAUSAL, bool DROPOUT, bool SPARSE, bool KB = false>
__global__ __launch_bounds__((64 * waves<SPARSE, D>()), (wgs_per_cu<SPARSE, D>())) void fa_fwd_kernel(FwdArgs a) {
  static_assert(!KB || (DROPOUT && !SPARSE), "keep bits: dense dropout instantiations only");
  static_assert(!KB || kBC == 64, "keep-bit words cover 64-key tiles");
  using T = MTile<D, kBC>;
  constexpr int kWaves = waves<SPARSE, D>();
  constexpr int kBR = rows_per_wg<SPARSE, D>();
  constexpr int kNS = 2 * (D / 16);  // S^T products per tile (two 32-key tiles x D/16 k-steps)
  constexpr int kNO = 4 * (D / 32);  // O^T products per tile (four 16-key slices x D/32 tiles)
  constexpr int kPF = 3;             // LDS operand reads in flight (products ahead)
  // 1 KB blocks of a K or V tile per wave (wave w loads blocks w, w + kWaves,
  // ...; with fewer blocks than a multiple of kWaves the last round is
  // partial), and tile loads per wave per tile step
  constexpr int kPer = (T::kBlocks + kWaves - 1) / kWaves;
  constexpr int kLoads = 2 * kPer;
  static_assert(kWaves == 4 || kLoads == 2 || kLoads == 4, "softmax-phase load spreading assumes 2 or 4 loads");
  static_assert(kNS % kLoads == 0 && kNS / kLoads >= 2, "product-phase load spreading");
  __shared__ __attribute__((aligned(1024))) uint16_t ks[2][T::kElems];
  __shared__ __attribute__((aligned(1024))) uint16_t vs[2][T::kElems];
  // block-sparse: the key tiles the workgroup visits (in order; the flags
  // are all 1: one mask row per workgroup)
  __shared__ uint16_t tlist[SPARSE ? kMaxSparseTiles : 1];
  __shared__ uint8_t tflag[SPARSE ? kMaxSparseTiles : 1];
  __shared__ int tcount[SPARSE ? 1 : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, known uniform
  const int h2 = lane >> 5;
  const int l32 = lane & 31;

  // Workgroup -> (b, h, query block).  Heads vary fastest so that, with the
  // round-robin dispatch over the 8 XCDs, every query block of one head lands
  // on the same XCD (K/V reuse in its L2) whenever B*H is a multiple of 8.
  // Causal: the longest query blocks (last rows) are dispatched first.  (Two
  // heads at a time per XCD, as the key-side backward does, cut the fetched
  // bytes at B 4, H 8, N 4096, d 128 causal from 197 to 145 MB but ran 2%
  // slower: the longest-first order matters more here.)
  const int BH = a.B * a.H;
  const int bh = blockIdx.x % BH;
  const int rank = blockIdx.x / BH;
  const int b = bh / a.H;
  const int h = bh % a.H;
  const int qb = CAUSAL ? a.nqb - 1 - rank : rank;
  int start, L;
  seq_bounds(a.cu, b, a.B, a.N, start, L);
  const int q0 = qb * kBR;
  if (q0 >= L) return;

  const int64_t ld = a.ld;
  const uint32_t row_bytes = (uint32_t)ld * 2;
  const uint16_t* kbase = a.k + (int64_t)start * ld + (int64_t)h * D;
  const uint16_t* vbase = a.v + (int64_t)start * ld + (int64_t)h * D;
  const int kv_end = CAUSAL ? min(L, q0 + kBR) : L;
  const int ntiles = (kv_end + kBC - 1) / kBC;

  const int qw = q0 + 32 * w;  // first query of this wave
  const int qi = qw + l32;     // query owned by this lane

  // keep-bit store: this head's words through a buffer descriptor; lane half
  // h2 writes word h2 of its query (rows past the end get an offset outside
  // the buffer, so their stores are dropped)
  const __amdgpu_buffer_rsrc_t kbr =
      KB ? make_rsrc(a.kbits + (int64_t)bh * a.nkt * 2 * a.kbn, (uint32_t)((uint64_t)a.nkt * 2 * a.kbn * 4))
         : make_rsrc(nullptr, 0u);
  const uint32_t kb_off = KB && qi < L ? (uint32_t)(h2 * a.kbn + qi) * 4u : 0x80000000u;

  // Q fragment: B operand of S^T = K Q^T (column = query, K slice = head dim);
  // rows past the end read as zeros.
  u32x4 qf[D / 16];
  {
    // a wave can start past the end of a ragged sequence: then its range is
    // empty and every load returns zero
    const int rows = max(0, min(32, L - qw));
    const uint32_t bytes = rows > 0 ? (uint32_t)(rows - 1) * row_bytes + D * 2 : 0u;
    const __amdgpu_buffer_rsrc_t qr = make_rsrc(a.q + (int64_t)(start + min(qw, L - 1)) * ld + (int64_t)h * D, bytes);
    const uint32_t off = (uint32_t)l32 * row_bytes + 16 * h2;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) qf[s] = buffer_load16(qr, off + 32 * s);
    // Consume the fragment here so the compiler's own wait for these loads
    // happens now and not inside the tile loop (where it would also wait for
    // the asynchronous K/V tile loads).
#pragma unroll
    for (int s = 0; s < D / 16; ++s) asm volatile("" : "+v"(qf[s]));
  }

  const uint32_t ks0 = lds_addr(ks), vs0 = lds_addr(vs);
  // Direct HBM -> LDS loads of one K or V tile: wave w issues blocks w,
  // w + kWaves, ... of it.
  auto issue = [&](const uint16_t* base, uint32_t lds, int j0) {
    const int rows = min(kBC, L - j0);
    const uint32_t bytes = (uint32_t)(rows - 1) * row_bytes + D * 2;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(base + (int64_t)j0 * ld, bytes);
#pragma unroll
    for (int u = 0; u < kPer; ++u)
      if (u * kWaves + w < T::kBlocks) T::load(r, lds, row_bytes, u * kWaves + w, lane);
  };

  f32x16 oacc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) oacc[dt] = f32x16{};
  float m_run = -INFINITY;  // reference max, in units of log2 (scores * scale * log2 e)
  float l_run = 0.f;        // this lane's share of the row sum
  f32x16 sacc[2];           // S^T of the tile being prepared (two 32-key halves)
  u32x4 pf[4];              // P^T of the tile being accumulated, as B operands

  const uint32_t ob0 = T::opnd_base(lane, 0), ob1 = T::opnd_base(lane, 1);
  const uint32_t tb0 = T::tr_base(lane, 0), tb1 = T::tr_base(lane, 1);

  // Last tile this wave needs: causal waves stop at the tile holding their
  // last query; waves that start past a ragged end need none.
  const int last = qw >= L ? -1 : (CAUSAL ? min(ntiles - 1, (qw + 31) / kBC) : ntiles - 1);

  // S^T = K Q^T of tile t into sacc, K operands read kPF products ahead.
  auto s_products = [&](int t) {
    uint32_t k0 = ks0 + (t & 1) * T::kBytes + ob0, k1 = ks0 + (t & 1) * T::kBytes + ob1;
    asm volatile("" : "+v"(k0), "+v"(k1));
    auto kread = [&](int i) {  // product i: key half i & 1, k-step i >> 1
      const int s = i >> 1;
      return lds_read16_at(((s & 1) ? k1 : k0) + T::opnd_off(i & 1, s));
    };
    sacc[0] = f32x16{};
    sacc[1] = f32x16{};
    u32x4 kb[kNS];
#pragma unroll
    for (int i = 0; i < kPF; ++i) kb[i] = kread(i);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < kNS; ++i) {
      sacc[i & 1] = mfma32<BF16>(kb[i], qf[i >> 1], sacc[i & 1]);
      if (i + kPF < kNS) kb[i + kPF] = kread(i + kPF);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Matrix phase of tile t: O^T += V^T P^T of tile t (if the wave needs it)
  // interleaved with S^T of tile t + 1 (if needed), LDS operands read kPF
  // products ahead.  The P^T registers are already the B operand (the key
  // order inside each 16-key slice is permuted and V^T is read with the
  // same permutation).
  auto m_phase = [&](int t, bool do_s, auto&& hook) __attribute__((always_inline)) {
    // the matrix phase issues ahead of the other group's softmax on the SIMD
    __builtin_amdgcn_s_setprio(1);
    if (do_s) {
      uint32_t k0 = ks0 + ((t + 1) & 1) * T::kBytes + ob0, k1 = ks0 + ((t + 1) & 1) * T::kBytes + ob1;
      uint32_t v0 = vs0 + (t & 1) * T::kBytes + tb0, v1 = vs0 + (t & 1) * T::kBytes + tb1;
      asm volatile("" : "+v"(k0), "+v"(k1), "+v"(v0), "+v"(v1));
      auto kread = [&](int i) {
        const int s = i >> 1;
        return lds_read16_at(((s & 1) ? k1 : k0) + T::opnd_off(i & 1, s));
      };
      auto vread = [&](int j) {  // product j: key slice j / (D/32), head-dim tile j % (D/32)
        const uint32_t o = T::tr_off(j / (D / 32), j % (D / 32));
        const u32x2 lo = lds_read_tr_at(v0 + o), hi = lds_read_tr_at(v1 + o);
        return u32x4{lo[0], lo[1], hi[0], hi[1]};
      };
      static_assert(kNS == kNO, "the two product streams are interleaved one to one");
      f32x16 s0 = f32x16{}, s1 = f32x16{};
      u32x4 kb[kNS], vb[kNO];
#pragma unroll
      for (int i = 0; i < kPF; ++i) {
        vb[i] = vread(i);
        kb[i] = kread(i);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < kNS; ++i) {
        oacc[i % (D / 32)] = mfma32<BF16>(vb[i], pf[i / (D / 32)], oacc[i % (D / 32)]);
        if (i & 1)
          s1 = mfma32<BF16>(kb[i], qf[i >> 1], s1);
        else
          s0 = mfma32<BF16>(kb[i], qf[i >> 1], s0);
        if (i + kPF < kNS) {
          vb[i + kPF] = vread(i + kPF);
          kb[i + kPF] = kread(i + kPF);
        }
        if (i % (kNS / kLoads) == 1) hook(i / (kNS / kLoads));
        __builtin_amdgcn_sched_barrier(0);
      }
      sacc[0] = s0;
      sacc[1] = s1;
    } else {
      uint32_t v0 = vs0 + (t & 1) * T::kBytes + tb0, v1 = vs0 + (t & 1) * T::kBytes + tb1;
      asm volatile("" : "+v"(v0), "+v"(v1));
      auto vread = [&](int j) {
        const uint32_t o = T::tr_off(j / (D / 32), j % (D / 32));
        const u32x2 lo = lds_read_tr_at(v0 + o), hi = lds_read_tr_at(v1 + o);
        return u32x4{lo[0], lo[1], hi[0], hi[1]};
      };
      u32x4 vb[kNO];
#pragma unroll
      for (int j = 0; j < kPF; ++j) vb[j] = vread(j);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < kNO; ++j) {
        oacc[j % (D / 32)] = mfma32<BF16>(vb[j], pf[j / (D / 32)], oacc[j % (D / 32)]);
        if (j + kPF < kNO) vb[j + kPF] = vread(j + kPF);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // keep bits of the last vector phase, stored by kb_flush after the slot's
  // barrier: a store issued just before a full vmcnt wait would stall on its
  // write acknowledgement
  uint32_t kb_word = 0;
  int kb_tile = 0;
  auto kb_flush = [&]() __attribute__((always_inline)) {
    if constexpr (KB)
      __builtin_amdgcn_raw_buffer_store_b32(kb_word, kbr, kb_off, (uint32_t)kb_tile * 8u * (uint32_t)a.kbn, 0);
  };

  // Vector phase of tile t: mask, online softmax of sacc (register r of key
  // half kt holds key t*kBC + kt*32 + 8*(r/4) + 4*h2 + r%4), dropout, and the
  // P^T operands of the next matrix phase.
  auto v_phase = [&](int t, bool may_mask, bool skip, auto&& hook) __attribute__((always_inline)) {
    // hook(u) for each of the kLoads tile loads, spread over four points
    auto at = [&](int point) {
      if constexpr (kLoads == 4) hook(point);
      else if (point % 2 == 0) hook(point / 2);
    };
    at(0);
    const int j0 = t * kBC;
    if (may_mask && ((CAUSAL && j0 + kBC - 1 > qw) || j0 + kBC > L)) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kj = j0 + kt * 32 + 8 * (r >> 2) + 4 * h2 + (r & 3);
          if ((CAUSAL && kj > qi) || kj >= L) sacc[kt][r] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kt][r]);
    mx = halves_max(mx) * a.scale_log2;
    // block-sparse: a tile listed for the other mask row only contributes
    // nothing (no max update, every probability 0)
    if constexpr (SPARSE) mx = skip ? -INFINITY : mx;
    at(1);
    const bool grow = mx > m_run + kRescaleLog2;
    if (__builtin_amdgcn_ballot_w64(grow)) {
      // rare: keep it a branch (the compiler would otherwise speculate the
      // rescale of the whole accumulator into every tile)
      asm volatile("" ::: "memory");
      const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - mx) : 1.f;
      m_run = grow ? mx : m_run;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) oacc[dt] *= alpha;
    }
    float m_use = m_run == -INFINITY ? 0.f : m_run;
    if constexpr (SPARSE) m_use = skip ? INFINITY : m_use;
    float rs = 0.f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kt][r], a.scale_log2, -m_use));
        rs += p;
        sacc[kt][r] = p;
      }
      at(2 + kt);
    }
    l_run += rs;
    if constexpr (DROPOUT) {
      uint32_t kbw[2] = {0u, 0u};  // keep bits of this lane's keys of key half kt (bit 16gp + 8u + e)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int gp = 0; gp < 2; ++gp) {
          // key groups 2gp, 2gp+1 of this half: words for keys 4*h2 .. 4*h2+3
          uint32_t kw[2][2];
          keep_words_pair(qi, j0 + kt * 32 + 16 * gp, h2, h, b, a.seed_lo, a.seed_hi, kw);
#pragma unroll
          for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const bool keep = keep16(kw[u][e >> 1], e & 1, a.drop_thresh);
              if (!keep) sacc[kt][4 * (2 * gp + u) + e] = 0.f;
              if constexpr (KB) kbw[kt] |= keep ? 1u << (16 * gp + 8 * u + e) : 0u;
            }
        }
      if constexpr (KB) {
        // the two lanes of a query hold alternate nibbles of each word (lane
        // half 1 the high ones): after the swap lane half h2 holds its
        // word h2 (keys 32*h2 .. 32*h2+31) as low nibbles in x, high in y
        uint32_t x = kbw[0], y = kbw[1];
        permlane32_swap(x, y);
        kb_word = x | (y << 4);
        kb_tile = t;
      }
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int kt = m >> 1;
      const int sub = (m & 1) * 8;
      pf[m] = u32x4{pack2<BF16>(sacc[kt][sub + 0], sacc[kt][sub + 1]),
                    pack2<BF16>(sacc[kt][sub + 2], sacc[kt][sub + 3]),
                    pack2<BF16>(sacc[kt][sub + 4], sacc[kt][sub + 5]),
                    pack2<BF16>(sacc[kt][sub + 6], sacc[kt][sub + 7])};
    }
  };

  // Two groups of four waves (one wave of each per SIMD) alternate a vector
  // phase V(t) (softmax of tile t) with a matrix phase M(t) (PV of tile t,
  // S of tile t + 1); the second group runs one phase behind the first, so
  // that on every SIMD one wave issues matrix products while the other does
  // its softmax.  Slots are separated by workgroup barriers: group 0 runs
  // V(t) in slot 2t and M(t) in slot 2t + 1, group 1 one slot later.  K and V
  // tiles are double-buffered (K(t), V(t) in buffer t % 2): K(t+2) and V(t+1)
  // are issued at the start of slot 2t + 1 (their buffers were last read in
  // slot 2t) and waited for at the end of slot 2t + 2.
  // Visited key tiles: all tiles 0 .. ntiles-1, or (block-sparse) the listed
  // ones.  Buffers follow the position k in that sequence; tile_at(k) is the
  // tile index.
  int n_list = ntiles;
  if constexpr (SPARSE) {
    if (w == 0) {
      const uint8_t* mrow = a.bmask + ((int64_t)b * a.H + h) * a.nb * a.nb;
      static_assert(!SPARSE || kBR == kMaskBlock, "one mask row per block-sparse workgroup");
      const int n = build_tile_list(mrow + (int64_t)(q0 / kMaskBlock) * a.nb, nullptr, 0, 1, ntiles, tlist, tflag,
                                    lane);
      if (lane == 0) tcount[0] = n;
    }
    __syncthreads();
    n_list = __builtin_amdgcn_readfirstlane(tcount[0]);
  }
  auto tile_at = [&](int k) __attribute__((always_inline)) -> int {
    if constexpr (SPARSE) return __builtin_amdgcn_readfirstlane(tlist[k]);
    else return k;
  };
  // ping-pong group (eight waves); the four-wave workgroups run every wave
  // as group 0 (no phase offset)
  const int grp = kWaves == 4 ? 0 : w / (kWaves / 2);
  auto skip_at = [&](int) __attribute__((always_inline)) -> bool { return false; };

  if (n_list > 0) {
    issue(kbase, ks0, tile_at(0) * kBC);
    issue(vbase, vs0, tile_at(0) * kBC);
  }
  if (n_list > 1) issue(kbase, ks0 + T::kBytes, tile_at(1) * kBC);
  wait_vmem();
  __syncthreads();
  // Load u (0 <= u < kLoads) of this wave's share of slot 2k + 1: blocks of
  // the K tile at position k+2 into buffer k % 2, then of the V tile at
  // position k+1 into buffer (k+1) % 2 (both buffers were last read in slot
  // 2k).  tk1, tk2 = tile indices at positions k+1, k+2 (or -1).
  // wv: the wave whose share is loaded (a group-1 wave also loads its
  // group-0 partner's when kG1Loads).
  auto load_part = [&](int k, int tk1, int tk2, int u, int wv) __attribute__((always_inline)) {
    constexpr int per = kPer;
    const bool isk = u < per;
    const int blk = (isk ? u : u - per) * kWaves + wv;
    if (T::kBlocks % kWaves != 0 && blk >= T::kBlocks) return;
    const int tt = isk ? tk2 : tk1;
    if (tt < 0) return;
    const int j0 = tt * kBC;
    const uint32_t bytes = (uint32_t)(min(kBC, L - j0) - 1) * row_bytes + D * 2;
    const __amdgpu_buffer_rsrc_t r = make_rsrc((isk ? kbase : vbase) + (int64_t)j0 * ld, bytes);
    const uint32_t lds = isk ? ks0 + (k & 1) * T::kBytes : vs0 + ((k + 1) & 1) * T::kBytes;
    T::load(r, lds, row_bytes, blk, lane);
  };
  auto tile_or_none = [&](int k) __attribute__((always_inline)) { return k < n_list ? tile_at(k) : -1; };
  auto no_hook = [](int) {};
  // The loop for one group G, whose wave-level schedule is fixed at compile
  // time: group 0 spreads its loads of slot 2k + 1 between the products of
  // M(k), group 1 through the softmax of V(k), so that no wave stalls on a
  // burst of load issues.  At d = 128 group 1 issues both groups' loads and
  // group 0's matrix phases issue none (2-4 % faster there; at d = 32 and 96,
  // where the softmax phase is the longer one, 3-6 % slower).
  constexpr bool kG1Loads = kWaves == 8 && D == 128;
  auto run = [&](auto G) __attribute__((always_inline)) {
    constexpr int g = decltype(G)::value;
    // the wave computes the visited tiles up to its last one: a prefix
    if (n_list > 0 && tile_at(0) <= last) s_products(0);
    if (g == 1) __syncthreads();  // slot 0: group 1 idle
    // Only the wave's last computed tile can hold masked keys (causal
    // diagonal or the ragged end), so the tiles before it run without mask
    // code.
    int k = 0;
    int tk = n_list > 0 ? tile_at(0) : -1;
    int tk1 = tile_or_none(1);
    for (; tk1 >= 0 && tk1 <= last; ++k) {
      const int tk2 = tile_or_none(k + 2);
      const bool skip = skip_at(k);
      auto loads = [&](int u) {
        load_part(k, tk1, tk2, u, w);
        if constexpr (kG1Loads) load_part(k, tk1, tk2, u, w - 4);
      };
      if constexpr (g == 1) v_phase(tk, false, skip, loads);
      else v_phase(tk, false, skip, no_hook);
      if (g == 0 && k > 0) wait_vmem();
      __syncthreads();
      kb_flush();
      if constexpr (g == 0 && !kG1Loads) m_phase(k, true, loads);
      else m_phase(k, true, no_hook);
      if (g == 1) wait_vmem();
      __syncthreads();
      tk = tk1;
      tk1 = tk2;
    }
    // The wave's last computed tile, then the slots of tiles it does not
    // need (it still issues its share of their loads).
    for (; k < n_list; ++k) {
      const int tk2 = tile_or_none(k + 2);
      const bool mine = tk <= last;
      if (g == 1)
        for (int u = 0; u < kLoads; ++u) {
          load_part(k, tk1, tk2, u, w);
          if constexpr (kG1Loads) load_part(k, tk1, tk2, u, w - 4);
        }
      if (mine) v_phase(tk, true, skip_at(k), no_hook);
      if (g == 0 && k > 0) wait_vmem();
      __syncthreads();
      if (mine) kb_flush();
      if (g == 0 && !kG1Loads)
        for (int u = 0; u < kLoads; ++u) load_part(k, tk1, tk2, u, w);
      if (mine) m_phase(k, false, no_hook);
      if (g == 1) wait_vmem();
      __syncthreads();
      tk = tk1;
      tk1 = tk2;
    }
    if (g == 0) __syncthreads();  // slot 2 * n_list: group 0 idle
  };
  if (grp == 0)
    run(std::integral_constant<int, 0>{});
  else
    run(std::integral_constant<int, 1>{});

  // ---- epilogue
  const float l_tot = halves_sum(l_run);
  const float inv = l_tot > 0.f ? (DROPOUT ? a.drop_rescale : 1.f) / l_tot : 0.f;
  if (qi < L) {
    uint16_t* op = a.o + (int64_t)(start + qi) * a.H * D + (int64_t)h * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = dt * 32 + 8 * g + 4 * h2;
        const u32x2 pk = {pack2<BF16>(oacc[dt][4 * g + 0] * inv, oacc[dt][4 * g + 1] * inv),
                          pack2<BF16>(oacc[dt][4 * g + 2] * inv, oacc[dt][4 * g + 3] * inv)};
        *reinterpret_cast<u32x2*>(op + d0) = pk;
      }
    if (h2 == 0) a.lse[(int64_t)(start + qi) * a.H + h] = (m_run + log2f(l_tot)) * kLn2;
  }
}

template <int D, bool BF16, bool CAUSAL, bool DROPOUT>
hipError_t launch_fwd_t(FwdArgs args, hipStream_t stream) {
  const bool sparse = args.bmask != nullptr;
  const int br = sparse ? rows_per_wg<true, D>() : rows_per_wg<false, D>();
  args.nqb = (args.N + br - 1) / br;
  const int64_t nblocks = (int64_t)args.nqb * args.B * args.H;
  if (nblocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (sparse)
    hipLaunchKernelGGL((fa_fwd_kernel<D, BF16, CAUSAL, DROPOUT, true>), dim3((unsigned)nblocks),
                       dim3(64 * waves<true, D>()), 0, stream, args);
  else if (DROPOUT && args.kbits)
    hipLaunchKernelGGL((fa_fwd_kernel<D, BF16, CAUSAL, DROPOUT, false, DROPOUT>), dim3((unsigned)nblocks),
                       dim3(64 * waves<false, D>()), 0, stream, args);
  else
    hipLaunchKernelGGL((fa_fwd_kernel<D, BF16, CAUSAL, DROPOUT, false>), dim3((unsigned)nblocks),
                       dim3(64 * waves<false, D>()), 0, stream, args);
  return hipGetLastError();
}

template <int D, bool BF16>
hipError_t launch_fwd_d(const AttnShape& s, const FwdArgs& args, hipStream_t stream) {
  static_assert(D % 32 == 0 && D >= 32 && D <= 256, "head sizes: multiples of 32 up to 256");
  if (s.causal)
    return s.dropout ? launch_fwd_t<D, BF16, true, true>(args, stream)
                     : launch_fwd_t<D, BF16, true, false>(args, stream);
  return s.dropout ? launch_fwd_t<D, BF16, false, true>(args, stream)
                   : launch_fwd_t<D, BF16, false, false>(args, stream);
}

// Dropout keep mask of one head, N x N bytes: one thread per 8 consecutive
// columns of a row (one Philox block).
__global__ __launch_bounds__(256) void fa_dropout_mask_kernel(uint8_t* keep, int b, int h, int N,
                                                              uint32_t thresh, uint32_t seed_lo,
                                                              uint32_t seed_hi) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int groups = (N + 7) / 8;
  if (t >= (int64_t)N * groups) return;
  const int i = (int)(t / groups);
  const int j8 = (int)(t % groups) * 8;
  const Philox4 r = philox4x32_10((uint32_t)i, (uint32_t)j8 >> 3, (uint32_t)h, (uint32_t)b, seed_lo, seed_hi);
  const uint32_t words[4] = {r.x, r.y, r.z, r.w};
  for (int e = 0; e < 8 && j8 + e < N; ++e)
    keep[(int64_t)i * N + j8 + e] = keep16(words[e >> 1], e & 1, thresh) ? 1 : 0;
}

}  // namespace

hipError_t launch_forward(const AttnShape& s, const void* q, const void* k, const void* v, void* o,
                          float* lse, hipStream_t stream) {
  FwdArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<uint16_t*>(o);
  a.lse = lse;
  a.cu = s.cu;
  a.ld = s.ld;
  a.B = s.B;
  a.H = s.H;
  a.N = s.N;
  a.nqb = 0;  // set by the launcher from the workgroup size of the instance
  a.scale_log2 = s.scale * kLog2e;
  a.drop_thresh = s.drop_thresh;
  a.drop_rescale = s.drop_rescale;
  a.seed_lo = (uint32_t)s.seed;
  a.seed_hi = (uint32_t)(s.seed >> 32);
  a.bmask = s.bmask;
  a.nb = s.nb;
  a.kbits = s.dropout ? s.keep_bits : nullptr;
  a.nkt = (s.N + 63) / 64;
  a.kbn = keep_bits_rows(s.N);
  switch (s.d) {
    case 32: return s.bf16 ? launch_fwd_d<32, true>(s, a, stream)
                           : launch_fwd_d<32, false>(s, a, stream);
    case 64: return s.bf16 ? launch_fwd_d<64, true>(s, a, stream)
                           : launch_fwd_d<64, false>(s, a, stream);
    case 96: return s.bf16 ? launch_fwd_d<96, true>(s, a, stream)
                           : launch_fwd_d<96, false>(s, a, stream);
    case 128: return s.bf16 ? launch_fwd_d<128, true>(s, a, stream)
                            : launch_fwd_d<128, false>(s, a, stream);
    case 160: return s.bf16 ? launch_fwd_d<160, true>(s, a, stream)
                            : launch_fwd_d<160, false>(s, a, stream);
    case 192: return s.bf16 ? launch_fwd_d<192, true>(s, a, stream)
                            : launch_fwd_d<192, false>(s, a, stream);
    default: return s.bf16 ? launch_fwd_d<256, true>(s, a, stream)
                           : launch_fwd_d<256, false>(s, a, stream);
  }
}

hipError_t launch_dropout_mask(uint8_t* keep, int b, int h, int N, uint32_t thresh, uint64_t seed,
                               hipStream_t stream) {
  const int64_t work = (int64_t)N * ((N + 7) / 8);
  const int64_t nblocks = (work + 255) / 256;
  if (nblocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(fa_dropout_mask_kernel, dim3((unsigned)nblocks), dim3(256), 0, stream, keep, b, h, N,
                     thresh, (uint32_t)seed, (uint32_t)(seed >> 32));
  return hipGetLastError();
}

}  // namespace fa
