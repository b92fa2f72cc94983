// fa_kernels.hip -- attention forward kernels for gfx950 (MI355X, CDNA4).
//
// What is computed: O = softmax(scale * Q K^T [+ causal mask]) V and lse = ln sum_j exp(scale * q.k_j),
// one (batch, head, 128-query tile) per workgroup, walking the K/V tiles with a running row maximum and
// running exponential sum so that the score matrix only ever exists as a register tile.
//   * Formula and tiling: page "FlashAttention：让长文本推理不再"卡显存"" (ai6s.net/6a0d42d8...),
//     sections "Attention 的显存黑洞" and "1. 分块计算（Tiling）".
//   * Running (m, l) update: same page, section "2. 在线归一化（Online Softmax）".  The page leaves
//     the output update implicit; the accumulator is multiplied by the same exp(m_old - m_new) as l and
//     divided by l at the end, the reading under which tiles reproduce the global softmax.
//   * lse output [B, H, N]: page ai6s.net/6a140d07..., section "第二层：数值稳定性增强".
//   * Causal diagonal skipping: page hwcomputing.csdn.net/6a0d4681..., section "Causal Mask的实现差异",
//     mode 2, with the exact rule "K tile visited iff its first key <= the tile's last query" and an
//     element mask (key > query) on the tiles that straddle the diagonal.
//   * Q tiles outer, K/V tiles inner, K/V re-read per Q tile: page hwcomputing.csdn.net/6a0d4681...,
//     section "分块策略：不是越大越好", constraint 2.
//
// gfx950 design (16-bit inputs):
//   * 4 waves x 32 queries = 128 queries per workgroup (8 waves, 256 queries, for the paired whole
//     causal problem); K/V tiles of 64 keys.
//   * MFMA v_mfma_f32_16x16x32_{bf16,f16}.  The kernel computes S^T = K Q^T and O^T = V^T P^T, so a
//     lane's accumulator registers all belong to one query (lane % 16): the softmax rescale is a
//     per-lane scalar, row reductions are in-lane plus two cross-lane steps, and the exponentiated
//     S^T registers are already laid out as the B operand of the P.V product (no LDS round trip).
//   * Q stays in VGPRs for the whole workgroup (B operand of S^T = K Q^T).
//   * K/V: global_load_lds_dwordx4 straight into a 2-stage LDS ring; the 16-byte chunk XOR swizzle is
//     applied on the global side (each lane fetches the chunk that belongs at its LDS slot).
//   * V^T operand: ds_read_b64_tr_b16 (transposing LDS read) from the row-major V tile.
//   * exp2 with scale*log2(e) folded into one FMA, against a reference maximum that is only moved when
//     needed: P is computed against the current reference, and only when some lane's partial sum shows a
//     probability above 2^64 (bf16; 2^14 for fp16), i.e. a new maximum far above the reference, or on a
//     wave's first active tile, is the row maximum taken, the state rescaled and P recomputed.  Exact up
//     to rounding either way.
//   * Row sums: l (for lse) in fp32 from the unrounded P; the normaliser of O from the P.V MFMA itself
//     against an all-ones operand, i.e. the sum of P exactly as rounded for the P.V product.
//   * Causal: per-wave skip of K tiles wholly above the wave's queries; element mask only on tiles
//     crossing the diagonal or the sequence end.
//   * Workgroup -> (head, Q tile) order: every XCD takes a contiguous run of heads (its L2 then holds
//     those heads' K/V), heaviest causal Q tiles first.  For the whole causal problem a workgroup runs
//     a pair of Q tiles of one head, the heaviest and the lightest remaining (equal work per pair), as
//     one stream of K/V tiles: the light tile's first K/V tile and its Q are fetched during the heavy
//     tile's last step.  Packed variable-length batches spread each sequence's heads over the XCDs.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

// fp32 kernel: deferred rescale threshold, in log2 units (probabilities stay below 2^8 before renormalising)
constexpr float kRescaleThreshold = 8.0f;
// 16-bit kernels: a lane's partial sum of 16 probabilities above this limit means some probability may
// exceed it, and the reference maximum moves.  P is rounded to the input type for the P.V product, so the
// limit keeps P representable there: 2^14 for fp16 (largest finite 65504); 2^64 for bf16, whose exponent
// range is fp32's (O, u and l accumulate in fp32: 2^16 keys x 2^64 x |v| stays far from overflow).
template <bool IS_BF16>
__device__ constexpr float part_limit() { return IS_BF16 ? 18446744073709551616.0f : 16384.0f; }
__device__ __forceinline__ float quad_max(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// ------------------------------------------------------------------------------------------------
// 16-bit inputs (bf16 / fp16)
// ------------------------------------------------------------------------------------------------
template <int D, int NW_ = 4>
struct Tile16 {
  static constexpr int NW = NW_;            // waves per workgroup
  static constexpr int QW = 32;             // queries per wave
  static constexpr int BM = NW * QW;        // queries per workgroup
  static constexpr int BN = 64;             // keys per K/V tile
  static constexpr int QG = QW / 16;        // 16-query groups per wave
  static constexpr int DC = D / 32;         // 32-wide d chunks (k dimension of S^T = K Q^T)
  static constexpr int DT = D / 16;         // 16-wide d tiles (rows of O^T)
  static constexpr int KT = BN / 16;        // 16-key tiles (rows of S^T)
  static constexpr int KC = BN / 32;        // 32-key chunks (k dimension of O^T = V^T P^T)
  static constexpr int ROW_BYTES = D * 2;
  static constexpr int CHUNKS = D / 8;      // 16-byte chunks per row
  static constexpr int TILE_BYTES = BN * ROW_BYTES;
  static constexpr int LOADS = TILE_BYTES / (16 * 64 * NW);  // 16-byte DMA loads per lane per tensor
  __device__ static __forceinline__ int swz_k(int row) { return D == 128 ? (row & 15) : ((row >> 1) & 7); }
  __device__ static __forceinline__ int swz_v(int row) { return D == 128 ? ((row & 7) << 1) : (((row >> 1) & 3) << 1); }
};

// Where one workgroup's sequence lies: its query and key counts, the causal offset, the element offsets
// of its (b, h) rows in Q/O and K/V, and the index of its first row in lse.  For packed variable-length
// batches these come from the sequence's offsets; offsets outside [0, total] or decreasing leave the
// sequence untouched (skip), so no offset array can send an access out of the tensors.
struct SeqGeom {
  int Nq, Nkv;
  int64_t delta, window, q_base, kv_base, lse_base;
  bool skip;
};

template <bool CAUSAL, bool VARLEN>
__device__ __forceinline__ SeqGeom seq_geometry(const Params& p, int b, int h, int bh) {
  SeqGeom sg;
  if constexpr (VARLEN) {
    const int qs = p.cu_q[b], qe = p.cu_q[b + 1], ks = p.cu_k[b], ke = p.cu_k[b + 1];
    sg.skip = qs < 0 || qe < qs || qe > p.total_q || ks < 0 || ke < ks || ke > p.total_k;
    sg.Nq = qe - qs;
    sg.Nkv = ke - ks;
    sg.delta = CAUSAL ? (int64_t)sg.Nkv - sg.Nq : 0;  // the two ends aligned
    sg.window = -1;
    sg.q_base = (int64_t)qs * p.stride_s + h * p.stride_h_q;
    sg.kv_base = (int64_t)ks * p.stride_s + h * p.stride_h_k;
    sg.lse_base = (int64_t)h * p.total_q + qs;
  } else {
    sg.skip = false;
    sg.Nq = p.Nq;
    sg.Nkv = p.Nkv;
    sg.delta = p.delta;
    sg.window = p.window;
    sg.q_base = b * p.stride_b_q + h * p.stride_h_q;
    sg.kv_base = b * p.stride_b_k + h * p.stride_h_k + p.kv_start * p.stride_s;
    sg.lse_base = (int64_t)bh * p.Nq;
  }
  return sg;
}

template <int D, bool IS_BF16, bool CAUSAL, bool WINDOW, bool VARLEN, bool PAIR, int NWV>
__global__ __launch_bounds__(64 * NWV, 8 / NWV) void fa_fwd_16(Params p) {
  typedef Tile16<D, NWV> T;
  typedef Elem<IS_BF16> E;
  typedef typename E::vec8 vec8;
  // Two stages for K and two for V, as four separate LDS objects: with the stage fixed at compile
  // time the compiler can tell that reads of one stage do not depend on the DMA filling the other.
  __shared__ __attribute__((aligned(1024))) uint8_t ks0[T::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t ks1[T::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t vs0[T::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t vs1[T::TILE_BYTES];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;    // lane group 0..3
  const int li = lane & 15;   // index within the group

  int bh, qt, qt_b = -1;
  if constexpr (VARLEN) {
    unit_of_spread(blockIdx.x, p.n_qtiles, CAUSAL, bh, qt);
    if (bh >= p.B * p.H) return;  // padding head of the grid
  } else if constexpr (PAIR) {
    // pair r of a head: its heavy tile n-1-r, then its light tile r (one causal tile of each end, so
    // every pair has the same work)
    int r;
    unit_of(blockIdx.x, p.n_units, p.n_qtiles, false, bh, r);
    const int n_full = (p.Nq + T::BM - 1) / T::BM;
    qt = n_full - 1 - r;
    qt_b = r;  // the launcher pairs only an even number of tiles
  } else {
    unit_of(blockIdx.x, p.n_units, p.n_qtiles, CAUSAL, bh, qt);
  }
  const int b = bh / p.H, h = bh - (bh / p.H) * p.H;
  const SeqGeom sg = seq_geometry<CAUSAL, VARLEN>(p, b, h, bh);
  int q_wg = qt * T::BM;
  if (VARLEN && (sg.skip || q_wg >= sg.Nq)) return;  // a bad sequence, or a tile past its end
  const int Nq = sg.Nq, Nkv = sg.Nkv;
  const int64_t delta = sg.delta, window = sg.window;
  int q0 = q_wg + wave * T::QW;

  const uint16_t* __restrict__ qg_ptr = (const uint16_t*)p.q + sg.q_base;
  const uint8_t* __restrict__ kg_ptr = (const uint8_t*)p.k + 2 * sg.kv_base;
  const uint8_t* __restrict__ vg_ptr = (const uint8_t*)p.v + 2 * sg.kv_base;

  // ---- the chunk keys this workgroup visits: from the lowest key inside the window of its first query
  // (0 without a window) to the last key visible to its last query; tiles of BN keys from k_begin ----
  const int k_begin = WINDOW ? (int)min((int64_t)Nkv, max((int64_t)0, q_wg + delta - window)) : 0;
  const int k_last = CAUSAL ? (int)max((int64_t)-1, min((int64_t)Nkv - 1, q_wg + T::BM - 1 + delta)) : Nkv - 1;
  const int n_kt_a = k_last >= k_begin ? (k_last - k_begin) / T::BN + 1 : 0;
  // the light tile of a pair (PAIR: no window, every tile sees key 0)
  const int n_kt_b = qt_b >= 0 ? (int)min((int64_t)Nkv - 1, qt_b * T::BM + T::BM - 1 + delta) / T::BN + 1 : 0;
  const int n_kt = n_kt_a + n_kt_b;
  if (n_kt == 0) {  // no query of this workgroup sees any key of the chunk: O = 0, lse = -inf
    uint16_t* og = (uint16_t*)p.o + sg.q_base;
#pragma unroll
    for (int qg = 0; qg < T::QG; ++qg) {
      const int qi = q0 + 16 * qg + li;
      if (qi < Nq) {
#pragma unroll
        for (int dt = 0; dt < T::DT; ++dt) *(u32x2_t*)(og + qi * p.stride_s + 16 * dt + 4 * g) = u32x2_t{0u, 0u};
        if (g == 0) p.lse[sg.lse_base + qi] = kNegInf;
      }
    }
    return;
  }

  // ---- K/V tile DMA: buffer loads straight into LDS.  The (b, h) base and the valid byte range sit in
  // a buffer descriptor (rows past the sequence end read as zeros and are masked); each lane adds a
  // fixed offset -- the global chunk that belongs at its LDS slot, i.e. the XOR swizzle applied on the
  // global side -- and each tile a uniform one. ----
  const int row_bytes = (int)(2 * p.stride_s);
  const int span = (Nkv - 1) * row_bytes + T::ROW_BYTES;  // the host keeps this below 2^31
  const __amdgpu_buffer_rsrc_t kbuf = __builtin_amdgcn_make_buffer_rsrc((void*)kg_ptr, 0, span, kBufferFlags);
  const __amdgpu_buffer_rsrc_t vbuf = __builtin_amdgcn_make_buffer_rsrc((void*)vg_ptr, 0, span, kBufferFlags);
  // Load i of a lane fills 16-byte slot (i*NW + wave)*64 + lane of the tile, NW*64/CHUNKS rows below
  // load 0's; both swizzles depend on the row only through bits that step leaves alone, so one lane
  // offset per tensor serves every load and the step goes into the uniform offset.
  int voff_k, voff_v;
  {
    const int slot = wave * 64 + lane;
    const int row = slot / T::CHUNKS, pc = slot % T::CHUNKS;
    voff_k = row * row_bytes + ((pc ^ T::swz_k(row)) << 4);
    voff_v = row * row_bytes + ((pc ^ T::swz_v(row)) << 4);
  }
  const int load_step = (T::NW * 64 / T::CHUNKS) * row_bytes;
  // tile j of the workgroup's sequence of tiles: the first unit's tiles, then the light unit's
  auto key_of = [&](int j) __attribute__((always_inline)) { return k_begin + (j < n_kt_a ? j : j - n_kt_a) * T::BN; };
  auto issue_tile = [&](int j, uint8_t* kdst, uint8_t* vdst) {
    const int soff = key_of(j) * row_bytes;
#pragma unroll
    for (int i = 0; i < T::LOADS; ++i) {
      const int lds_off = (i * T::NW + wave) * 1024;  // wave-uniform base; lane lands at +16*lane
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kbuf, (lds_void_t*)(kdst + lds_off), 16, voff_k, soff + i * load_step, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vbuf, (lds_void_t*)(vdst + lds_off), 16, voff_v, soff + i * load_step, 0, 0);
    }
  };

  issue_tile(0, ks0, vs0);

  // ---- Q fragments (B operand of S^T = K Q^T): lane holds q[q0 + 16*qg + li][32*c + 8*g .. +7] ----
  vec8 qf[T::QG][T::DC];
  auto load_q = [&](int qbase) __attribute__((always_inline)) {
#pragma unroll
    for (int qg = 0; qg < T::QG; ++qg) {
      const int qrow = min(qbase + 16 * qg + li, Nq - 1);
#pragma unroll
      for (int c = 0; c < T::DC; ++c) {
        u32x4_t raw = *(const u32x4_t*)(qg_ptr + qrow * p.stride_s + 32 * c + 8 * g);
        raw ^= p.qsign;  // exact negation when scale < 0 (the exponent then uses |scale|)
        qf[qg][c] = __builtin_bit_cast(vec8, raw);
      }
    }
  };
  load_q(q0);

  const float cexp = p.c;  // |scale| * log2(e)
  float m_ref[T::QG], l_part[T::QG];
  f32x4_t oacc[T::QG][T::DT], uacc[T::QG];
#pragma unroll
  for (int qg = 0; qg < T::QG; ++qg) {
    m_ref[qg] = kNegInf;
    l_part[qg] = 0.f;
    uacc[qg] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dt = 0; dt < T::DT; ++dt) oacc[qg][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  // Per-lane LDS byte offsets of the fragment reads.  Both swizzles depend on the row only through
  // bits that a 16-row (K) or 32-row (V) step leaves alone, so each read is one of these per-lane
  // bases plus a constant (the row step), which goes into the instruction's offset field.
  int kb[T::DC], vb[T::DT];
#pragma unroll
  for (int c = 0; c < T::DC; ++c) kb[c] = li * T::ROW_BYTES + (((4 * c + g) ^ T::swz_k(li)) << 4);
#pragma unroll
  for (int dt = 0; dt < T::DT; ++dt) {
    const int vrow = 4 * g + (li >> 2);
    const int col = 16 * dt + 4 * (li & 3);  // element column of this lane's 4-element read
    vb[dt] = vrow * T::ROW_BYTES + (((col >> 3) ^ T::swz_v(vrow)) << 4) + (col & 7) * 2;
  }

  bool first_tile = true;  // wave-uniform: no tile processed yet (a window or chunk can skip the first ones)

  // One K/V tile: wait for its DMA, prefetch the next one into the other stage, compute.
  // The last tile is a separate compile-time variant (no prefetch, full wait) so that every wait on
  // the DMA counter is unconditional and the compiler adds none of its own before LDS reads.
  // epilogue of the current unit: O = acc / u, lse = (m + log2 l) ln 2; a row without any visible key
  // has u = l = 0 and gets O = 0, lse = -inf
  uint16_t* og_ptr = (uint16_t*)p.o + sg.q_base;
  auto finish = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int qg = 0; qg < T::QG; ++qg) {
      const float l = wave_sum_xor16_32(l_part[qg]);
      const float inv = uacc[qg][0] > 0.0f ? 1.0f / uacc[qg][0] : 0.0f;
      const int qi = q0 + 16 * qg + li;
      if (qi < Nq) {
#pragma unroll
        for (int dt = 0; dt < T::DT; ++dt) {
          const f32x4_t o = oacc[qg][dt] * inv;
          u32x2_t w = {E::pack2(o[0], o[1]), E::pack2(o[2], o[3])};
          *(u32x2_t*)(og_ptr + qi * p.stride_s + 16 * dt + 4 * g) = w;
        }
        if (g == 0) p.lse[sg.lse_base + qi] = (m_ref[qg] + __builtin_log2f(l)) * kLn2;
      }
    }
  };

  const std::integral_constant<bool, false> stay;
  const std::integral_constant<bool, true> switch_c;
  auto step = [&](int j, const uint8_t* ks, const uint8_t* vs, uint8_t* kn, uint8_t* vn, auto last_c,
                  auto sw_c) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // this wave's share of tile j has landed
    lds_barrier();  // tile j is in LDS for every wave, and every wave is done with tile j-1
    if constexpr (!decltype(last_c)::value) issue_tile(j + 1, kn, vn);  // into tile j-1's stage

    const int key0 = key_of(j);  // first chunk key of tile j
    // the last tile of the heavy unit of a pair: the light unit's Q is loaded once S^T no longer needs
    // the heavy unit's (the state moves over to the light unit after this step)
    constexpr bool switch_unit = decltype(sw_c)::value;
    // the wave's 32 queries see some key of this tile (causal: its first key is not after the last
    // query's position; window: its last key is not before the first query's window)
    const bool active = (!CAUSAL || key0 <= q0 + T::QW - 1 + delta) && (!WINDOW || key0 + T::BN - 1 >= q0 + delta - window);
    if (active) {
      // ---- S^T = K Q^T : s[qg][kt] holds keys key0 + 16*kt + 4*g + r for query q0 + 16*qg + li ----
      // the K fragments of 16-key tile kt+1 are read while tile kt's MFMAs run
      f32x4_t s[T::QG][T::KT];
      auto k_frag = [&](int kt, int c) { return *(const vec8*)(ks + kb[c] + 16 * kt * T::ROW_BYTES); };
      vec8 kf[T::DC], kf_next[T::DC];
#pragma unroll
      for (int c = 0; c < T::DC; ++c) kf_next[c] = k_frag(0, c);
#pragma unroll
      for (int kt = 0; kt < T::KT; ++kt) {
#pragma unroll
        for (int c = 0; c < T::DC; ++c) kf[c] = kf_next[c];
        if (kt + 1 < T::KT) {
#pragma unroll
          for (int c = 0; c < T::DC; ++c) kf_next[c] = k_frag(kt + 1, c);
        }
        // keeps the scheduler from moving the reads above back down next to their MFMAs
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int qg = 0; qg < T::QG; ++qg) s[qg][kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < T::DC; ++c)
#pragma unroll
          for (int qg = 0; qg < T::QG; ++qg) s[qg][kt] = E::mfma(kf[c], qf[qg][c], s[qg][kt]);
      }
      if constexpr (switch_unit) load_q(qt_b * T::BM + wave * T::QW);

      // ---- mask, online softmax, P ----
      const bool need_mask = (CAUSAL && key0 + T::BN - 1 > q0 + delta) || (key0 + T::BN > Nkv) ||
                             (WINDOW && key0 < q0 + T::QW - 1 + delta - window);
      if (need_mask) {
        keep_branch();
        // the wave's first query position minus key0 (and minus the window), once per tile in 64 bits,
        // clamped: the slots span fewer than 64 keys, so values past +-512 hide the same slots
        const int dq0 = CAUSAL ? (int)max((int64_t)-512, min((int64_t)512, q0 + delta - key0)) : 0;
        const int dw0 = WINDOW ? (int)max((int64_t)-512, min((int64_t)512, q0 + delta - window - key0)) : 0;
        const int kend = min(512, Nkv - key0);  // slots from kend on lie past the chunk
#pragma unroll
        for (int qg = 0; qg < T::QG; ++qg) {
          // visible slots 16*kt + r (key key0 + 16*kt + 4*g + r) of this lane's query: up to hi (causal
          // edge or chunk end) and, with a window, from lo; keys before the chunk are never in a tile
          const int hi = (CAUSAL ? min(kend - 1, dq0 + 16 * qg + li) : kend - 1) - 4 * g;
          const int lo = WINDOW ? dw0 + 16 * qg + li - 4 * g : 0;
#pragma unroll
          for (int kt = 0; kt < T::KT; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (16 * kt + r > hi || (WINDOW && 16 * kt + r < lo)) s[qg][kt][r] = kNegInf;
        }
      }
      // P = exp2(c s - m_ref) against the current reference maximum; valid while no probability exceeds
      // the dtype's limit, which each lane checks through its partial sums.  Otherwise (and on a wave's first tile)
      // the reference moves to the running maximum first and P is recomputed.
      uint32_t pf[T::QG][T::KC][4];
      float part[T::QG];
      auto expo = [&](int qg) __attribute__((always_inline)) {
        const float neg_m = -m_ref[qg];
        float acc = 0.f;
#pragma unroll
        for (int kt = 0; kt < T::KT; ++kt) {
          float pv[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) pv[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qg][kt][r], cexp, neg_m));
          acc += (pv[0] + pv[1]) + (pv[2] + pv[3]);
          const int kc = kt >> 1, half = kt & 1;
          pf[qg][kc][2 * half + 0] = E::pack2(pv[0], pv[1]);
          pf[qg][kc][2 * half + 1] = E::pack2(pv[2], pv[3]);
        }
        part[qg] = acc;
      };
      const bool first = first_tile;  // the wave's first active tile sets the reference maximum
      first_tile = false;
      // each 16-query group moves its reference only when one of its lanes needs it
      bool slow[T::QG];
#pragma unroll
      for (int qg = 0; qg < T::QG; ++qg) {
        slow[qg] = first;
        if (!first) {
          expo(qg);
          slow[qg] = __builtin_amdgcn_ballot_w64(part[qg] > part_limit<IS_BF16>()) != 0;
        }
      }
#pragma unroll
      for (int qg = 0; qg < T::QG; ++qg) {
        if (slow[qg]) {
          keep_branch();
          float mx = kNegInf;
#pragma unroll
          for (int kt = 0; kt < T::KT; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[qg][kt][r]);
          mx = quad_max(mx);
          // a row that has seen no visible key yet takes 0 as its reference (its sums stay 0 and any
          // reference is valid until a probability would exceed the limit, which the check above catches)
          float m_new = fmaxf(m_ref[qg], mx * cexp);
          if (m_new == kNegInf) m_new = 0.0f;
          const float alpha = __builtin_amdgcn_exp2f(m_ref[qg] - m_new);
          l_part[qg] *= alpha;
          uacc[qg] *= alpha;
#pragma unroll
          for (int dt = 0; dt < T::DT; ++dt) oacc[qg][dt] *= alpha;
          m_ref[qg] = m_new;
          expo(qg);
        }
      }
#pragma unroll
      for (int qg = 0; qg < T::QG; ++qg) l_part[qg] += part[qg];

      // ---- O^T += V^T P^T ----
      // V^T fragments of (kc, dt) via transposing reads: lanes 4e..4e+3 of each 16-lane group address
      // row e and lane li receives column li of those rows; read VA fragments ahead of their MFMAs
      auto v_frag = [&](int f) {
        const int kc = f / T::DT, dt = f % T::DT;
        const uint8_t* a0 = vs + vb[dt] + 32 * kc * T::ROW_BYTES;
        const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)a0);
        const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(a0 + 16 * T::ROW_BYTES));
        u32x4_t w = {__builtin_bit_cast(u32x2_t, lo)[0], __builtin_bit_cast(u32x2_t, lo)[1],
                     __builtin_bit_cast(u32x2_t, hi)[0], __builtin_bit_cast(u32x2_t, hi)[1]};
        return __builtin_bit_cast(vec8, w);
      };
      constexpr int NF = T::KC * T::DT, VA = 4;
      vec8 vring[VA];
#pragma unroll
      for (int f = 0; f < VA; ++f) vring[f] = v_frag(f);
      // u: the same MFMA against an all-ones operand sums P as rounded for the P.V product
#pragma unroll
      for (int kc = 0; kc < T::KC; ++kc)
#pragma unroll
        for (int qg = 0; qg < T::QG; ++qg) {
          u32x4_t w = {pf[qg][kc][0], pf[qg][kc][1], pf[qg][kc][2], pf[qg][kc][3]};
          uacc[qg] = E::mfma(E::ones(), __builtin_bit_cast(vec8, w), uacc[qg]);
        }
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const vec8 vf = vring[f % VA];
        if (f + VA < NF) vring[f % VA] = v_frag(f + VA);
        __builtin_amdgcn_sched_barrier(0);  // the same for the V^T reads
        const int kc = f / T::DT, dt = f % T::DT;
#pragma unroll
        for (int qg = 0; qg < T::QG; ++qg) {
          u32x4_t w = {pf[qg][kc][0], pf[qg][kc][1], pf[qg][kc][2], pf[qg][kc][3]};
          oacc[qg][dt] = E::mfma(vf, __builtin_bit_cast(vec8, w), oacc[qg][dt]);
        }
      }
    } else if constexpr (switch_unit) {
      load_q(qt_b * T::BM + wave * T::QW);
    }
  };

  const std::integral_constant<bool, false> more;
  const std::integral_constant<bool, true> last;
  if constexpr (PAIR) {
    // both units have an even number of tiles (the launcher pairs only then), so every tile j sits in
    // stage j % 2 and the light unit starts in stage 0; the heavy unit's last step prefetches the
    // light unit's first tile
    int j = 0;
    for (; j + 2 < n_kt_a; j += 2) {
      step(j, ks0, vs0, ks1, vs1, more, stay);
      step(j + 1, ks1, vs1, ks0, vs0, more, stay);
    }
    step(j, ks0, vs0, ks1, vs1, more, stay);
    step(j + 1, ks1, vs1, ks0, vs0, more, switch_c);  // loads the light unit's Q after its S^T
    j += 2;
    finish();
    q_wg = qt_b * T::BM;
    q0 = q_wg + wave * T::QW;
    first_tile = true;
#pragma unroll
    for (int qg = 0; qg < T::QG; ++qg) {
      m_ref[qg] = kNegInf;
      l_part[qg] = 0.f;
      uacc[qg] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int dt = 0; dt < T::DT; ++dt) oacc[qg][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    for (; j + 2 < n_kt; j += 2) {
      step(j, ks0, vs0, ks1, vs1, more, stay);
      step(j + 1, ks1, vs1, ks0, vs0, more, stay);
    }
    step(j, ks0, vs0, ks1, vs1, more, stay);
    step(j + 1, ks1, vs1, ks0, vs0, last, stay);
  } else {
    int j = 0;
    for (; j + 2 < n_kt; j += 2) {
      step(j, ks0, vs0, ks1, vs1, more, stay);
      step(j + 1, ks1, vs1, ks0, vs0, more, stay);
    }
    if (j + 2 == n_kt) {
      step(j, ks0, vs0, ks1, vs1, more, stay);
      step(j + 1, ks1, vs1, ks0, vs0, last, stay);
    } else {
      step(j, ks0, vs0, ks1, vs1, last, stay);
    }
  }
  finish();
}

// ------------------------------------------------------------------------------------------------
// fp32 inputs: the same S^T / O^T formulation on v_mfma_f32_16x16x4_f32 (fp32 end to end).
// ------------------------------------------------------------------------------------------------
template <int D>
struct Tile32 {
  static constexpr int NW = 4;
  static constexpr int QW = 32;
  static constexpr int BM = NW * QW;
  static constexpr int BN = 32;
  static constexpr int QG = QW / 16;
  static constexpr int DK = D / 4;       // k steps of S^T = K Q^T
  static constexpr int DT = D / 16;      // 16-wide d tiles of O^T
  static constexpr int KT = BN / 16;
  static constexpr int LD = D + 4;       // padded LDS row (floats)
};

template <int D, bool CAUSAL, bool WINDOW>
__global__ __launch_bounds__(256, 1) void fa_fwd_32(Params p) {
  typedef Tile32<D> T;
  __shared__ float ks[T::BN * T::LD];
  __shared__ float vs[T::BN * T::LD];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4, li = lane & 15;

  int bh, qt;
  unit_of(blockIdx.x, p.n_units, p.n_qtiles, CAUSAL, bh, qt);
  const int b = bh / p.H, h = bh - (bh / p.H) * p.H;
  const int Nq = p.Nq, Nkv = p.Nkv;
  const int64_t delta = p.delta, window = p.window;
  const int q_wg = qt * T::BM;
  const int q0 = q_wg + wave * T::QW;
  const float* qg_ptr = (const float*)p.q + b * p.stride_b_q + h * p.stride_h_q;
  const int64_t kv_base = b * p.stride_b_k + h * p.stride_h_k + p.kv_start * p.stride_s;
  const float* kg_ptr = (const float*)p.k + kv_base;
  const float* vg_ptr = (const float*)p.v + kv_base;
  const float qsign = p.qsign ? -1.0f : 1.0f;

  // Q^T fragments: lane holds q[q0 + 16*qg + li][4*kk + g]
  float qf[T::QG][T::DK];
#pragma unroll
  for (int qg = 0; qg < T::QG; ++qg) {
    const int qrow = min(q0 + 16 * qg + li, Nq - 1);
#pragma unroll
    for (int kk = 0; kk < T::DK; ++kk) qf[qg][kk] = qsign * qg_ptr[qrow * p.stride_s + 4 * kk + g];
  }
  // chunk keys visited: as in the 16-bit kernel (may be none: then O = 0, lse = -inf)
  const int k_begin = WINDOW ? (int)min((int64_t)Nkv, max((int64_t)0, q_wg + delta - window)) : 0;
  const int k_last = CAUSAL ? (int)max((int64_t)-1, min((int64_t)Nkv - 1, q_wg + T::BM - 1 + delta)) : Nkv - 1;
  const int n_kt = k_last >= k_begin ? (k_last - k_begin) / T::BN + 1 : 0;
  const float cexp = p.c;
  float m_ref[T::QG], l_part[T::QG];
  f32x4_t oacc[T::QG][T::DT];
#pragma unroll
  for (int qg = 0; qg < T::QG; ++qg) {
    m_ref[qg] = kNegInf;
    l_part[qg] = 0.f;
#pragma unroll
    for (int dt = 0; dt < T::DT; ++dt) oacc[qg][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  for (int j = 0; j < n_kt; ++j) {
    const int key0 = k_begin + j * T::BN;
    // stage K, V tile through registers (16-byte loads, padded rows; rows past the chunk repeat its
    // last row and are masked)
    for (int idx = threadIdx.x; idx < T::BN * (D / 4); idx += 256) {
      const int row = idx / (D / 4), c4 = idx % (D / 4);
      const int key = min(key0 + row, Nkv - 1);
      const float4 kv = *(const float4*)(kg_ptr + key * p.stride_s + 4 * c4);
      const float4 vv = *(const float4*)(vg_ptr + key * p.stride_s + 4 * c4);
      *(float4*)(ks + row * T::LD + 4 * c4) = kv;
      *(float4*)(vs + row * T::LD + 4 * c4) = vv;
    }
    __syncthreads();
    const bool active = (!CAUSAL || key0 <= q0 + T::QW - 1 + delta) && (!WINDOW || key0 + T::BN - 1 >= q0 + delta - window);
    if (active) {
      f32x4_t s[T::QG][T::KT];
#pragma unroll
      for (int kt = 0; kt < T::KT; ++kt) {
#pragma unroll
        for (int qg = 0; qg < T::QG; ++qg) s[qg][kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < T::DK; ++kk) {
          const float kf = ks[(16 * kt + li) * T::LD + 4 * kk + g];
#pragma unroll
          for (int qg = 0; qg < T::QG; ++qg) s[qg][kt] = __builtin_amdgcn_mfma_f32_16x16x4f32(kf, qf[qg][kk], s[qg][kt], 0, 0, 0);
        }
      }
      const bool need_mask = (CAUSAL && key0 + T::BN - 1 > q0 + delta) || (key0 + T::BN > Nkv) ||
                             (WINDOW && key0 < q0 + T::QW - 1 + delta - window);
#pragma unroll
      for (int qg = 0; qg < T::QG; ++qg) {
        const int qi = q0 + 16 * qg + li;
        if (need_mask) {
          const int hi = CAUSAL ? (int)max((int64_t)-1, min((int64_t)Nkv - 1, qi + delta)) : Nkv - 1;
          const int lo = WINDOW ? (int)min((int64_t)Nkv, max((int64_t)0, qi + delta - window)) : 0;
#pragma unroll
          for (int kt = 0; kt < T::KT; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int key = key0 + 16 * kt + 4 * g + r;
              if (key > hi || key < lo) s[qg][kt][r] = kNegInf;
            }
        }
        float mx = kNegInf;
#pragma unroll
        for (int kt = 0; kt < T::KT; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[qg][kt][r]);
        mx = wave_max_xor16_32(mx);
        const float mx_c = (mx == kNegInf) ? kNegInf : mx * cexp;
        const float m_cand = fmaxf(m_ref[qg], mx_c);
        const bool move = m_cand > m_ref[qg] + kRescaleThreshold;
        if (__builtin_amdgcn_ballot_w64(move) != 0) {
          const float m_new = move ? m_cand : m_ref[qg];
          // a row that stays put keeps its sums (also when it has seen no visible key: -inf - -inf)
          const float alpha = move ? __builtin_amdgcn_exp2f(m_ref[qg] - m_new) : 1.0f;
          l_part[qg] *= alpha;
#pragma unroll
          for (int dt = 0; dt < T::DT; ++dt) oacc[qg][dt] *= alpha;
          m_ref[qg] = m_new;
        }
        const float neg_m = -m_ref[qg];
#pragma unroll
        for (int kt = 0; kt < T::KT; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float x = __builtin_fmaf(s[qg][kt][r], cexp, neg_m);
            if (need_mask && s[qg][kt][r] == kNegInf) x = kNegInf;
            const float pv = __builtin_amdgcn_exp2f(x);
            s[qg][kt][r] = pv;
            l_part[qg] += pv;
          }
      }
      // O^T += V^T P^T, one k step per (kt, r): key slot g <-> key 16*kt + 4*g + r
#pragma unroll
      for (int kt = 0; kt < T::KT; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int vrow = 16 * kt + 4 * g + r;
#pragma unroll
          for (int dt = 0; dt < T::DT; ++dt) {
            const float vf = vs[vrow * T::LD + 16 * dt + li];
#pragma unroll
            for (int qg = 0; qg < T::QG; ++qg)
              oacc[qg][dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(vf, s[qg][kt][r], oacc[qg][dt], 0, 0, 0);
          }
        }
    }
    __syncthreads();
  }

  float* og_ptr = (float*)p.o + b * p.stride_b_q + h * p.stride_h_q;
#pragma unroll
  for (int qg = 0; qg < T::QG; ++qg) {
    const float l = wave_sum_xor16_32(l_part[qg]);
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;  // l = 0: no visible key, O = 0 and lse = -inf
    const int qi = q0 + 16 * qg + li;
    if (qi < Nq) {
#pragma unroll
      for (int dt = 0; dt < T::DT; ++dt) {
        const f32x4_t o = oacc[qg][dt] * inv;
        *(float4*)(og_ptr + qi * p.stride_s + 16 * dt + 4 * g) = make_float4(o[0], o[1], o[2], o[3]);
      }
      if (g == 0) p.lse[(int64_t)bh * Nq + qi] = (m_ref[qg] + __builtin_log2f(l)) * kLn2;
    }
  }
}

// ------------------------------------------------------------------------------------------------
// launchers
// ------------------------------------------------------------------------------------------------
template <int D, bool IS_BF16, bool CAUSAL, bool WINDOW, bool VARLEN = false, bool PAIR = false, int NWV = 4>
static hipError_t launch16(Params p, hipStream_t stream) {
  typedef Tile16<D, NWV> T;
  p.n_qtiles = (p.Nq + T::BM - 1) / T::BM;
  if (PAIR) p.n_qtiles = (p.n_qtiles + 1) / 2;  // pairs of tiles per head
  // packed sequences: heads spread over the XCDs, the grid padded to a multiple of 8 heads
  p.n_units = p.n_qtiles * (VARLEN ? (p.B * p.H + 7) / 8 * 8 : p.B * p.H);
  hipLaunchKernelGGL((fa_fwd_16<D, IS_BF16, CAUSAL, WINDOW, VARLEN, PAIR, NWV>), dim3(p.n_units), dim3(64 * NWV), 0,
                     stream, p);
  return hipGetLastError();
}

template <int D, bool CAUSAL, bool WINDOW>
static hipError_t launch32(Params p, hipStream_t stream) {
  typedef Tile32<D> T;
  p.n_qtiles = (p.Nq + T::BM - 1) / T::BM;
  p.n_units = p.n_qtiles * p.B * p.H;
  hipLaunchKernelGGL((fa_fwd_32<D, CAUSAL, WINDOW>), dim3(p.n_units), dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <int D, bool IS_BF16>
static hipError_t launch16_d(const Params& p, bool causal, hipStream_t stream) {
  if (!causal) return launch16<D, IS_BF16, false, false>(p, stream);
  if (p.window >= 0) return launch16<D, IS_BF16, true, true>(p, stream);
  // The whole causal problem (every query tile sees key 0): pairs of heavy and light tiles.  The pair
  // loop needs an even number of query tiles, each visiting an even number of 64-key tiles: the full
  // tiles do (BM is a multiple of 128), the last one does when the key count rounds up to an even
  // number of key tiles.  Pairs of 256-query tiles (8 waves) first, then of 128-query tiles.
  const bool whole = p.delta == 0 && p.Nq == p.Nkv && p.kv_start == 0;
  const bool even_keys = ((p.Nq + Tile16<D>::BN - 1) / Tile16<D>::BN) % 2 == 0;
  const auto pairs = [&](int bm) { return whole && even_keys && ((p.Nq + bm - 1) / bm) % 2 == 0; };
  if (pairs(Tile16<D, 8>::BM)) return launch16<D, IS_BF16, true, false, false, true, 8>(p, stream);
  if (pairs(Tile16<D, 4>::BM)) return launch16<D, IS_BF16, true, false, false, true, 4>(p, stream);
  return launch16<D, IS_BF16, true, false>(p, stream);
}

template <int D>
static hipError_t launch32_d(const Params& p, bool causal, hipStream_t stream) {
  if (!causal) return launch32<D, false, false>(p, stream);
  return p.window >= 0 ? launch32<D, true, true>(p, stream) : launch32<D, true, false>(p, stream);
}

// A window is only used with causal attention (the entry point rejects it otherwise).
hipError_t launch(const Params& p, int dtype, int d, bool causal, hipStream_t stream) {
  if (dtype == kDtypeBf16) return d == 128 ? launch16_d<128, true>(p, causal, stream) : launch16_d<64, true>(p, causal, stream);
  if (dtype == kDtypeFp16) return d == 128 ? launch16_d<128, false>(p, causal, stream) : launch16_d<64, false>(p, causal, stream);
  return d == 128 ? launch32_d<128>(p, causal, stream) : launch32_d<64>(p, causal, stream);
}

template <int D, bool IS_BF16>
static hipError_t launch_varlen_d(const Params& p, bool causal, hipStream_t stream) {
  return causal ? launch16<D, IS_BF16, true, false, true>(p, stream) : launch16<D, IS_BF16, false, false, true>(p, stream);
}

hipError_t launch_varlen(const Params& p, int dtype, int d, bool causal, hipStream_t stream) {
  if (dtype == kDtypeBf16)
    return d == 128 ? launch_varlen_d<128, true>(p, causal, stream) : launch_varlen_d<64, true>(p, causal, stream);
  return d == 128 ? launch_varlen_d<128, false>(p, causal, stream) : launch_varlen_d<64, false>(p, causal, stream);
}

int queries_per_workgroup(int dtype) { return dtype == kDtypeFp32 ? Tile32<64>::BM : Tile16<64>::BM; }

}  // namespace fa
