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
// Reference maximum (log2 units) of a row that has seen no visible key: exp2 of any visible logit minus it
// is +inf, which the limit check catches.
constexpr float kNoKeyRef = -1.0e30f;
template <bool IS_BF16>
__device__ constexpr float part_limit() { return IS_BF16 ? 18446744073709551616.0f : 16384.0f; }
__device__ __forceinline__ float quad_max(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

#ifdef FA_TILE_COUNT
// Test-only build (libfa_tilecount.so): every 16-bit forward workgroup records the K/V tiles it visits, so a
// test can hold them against the closed form of the visibility rule.  Record of block x (kTileRecInts ints):
// [0] b*H + h (the head slot), [1] queries per unit, [2] keys per tile, [3] queries per wave, [4] first query
// of the first unit, [5] tiles it streams, [6] first query of a pair's light unit or -1, [7] its tiles,
// [8 + w] tiles wave w computes on (both units), [16] waves, [17] 0 for fa_fwd_16, 1 for fa_fwd_16pp,
// [18] the row after the record's last real row (a unit's rows end there).
__device__ int* g_tile_rec = nullptr;
__device__ long long g_tile_rec_cap = 0;
#endif
[[maybe_unused]] constexpr int kTileRecInts = 24;
// (slots count from the launch's rec_base, rows from its q_row0: a call split into launches over row ranges
// records like one launch over all rows)
__device__ __forceinline__ void record_tiles_at(const Params& p, int slot, int kernel, int bh, int bm, int bn, int qw,
                                                int nw, int qa, int na, int qb, int nb, int wave, int lane, int n_act,
                                                int row_end) {
#ifdef FA_TILE_COUNT
  slot += p.rec_base;
  qa += p.q_row0;
  if (qb >= 0) qb += p.q_row0;
  int* rec = g_tile_rec;
  if (lane == 0 && rec != nullptr && (long long)slot < g_tile_rec_cap) {
    int* r = rec + (size_t)slot * kTileRecInts;
    if (wave == 0) {
      r[0] = bh;
      r[1] = bm;
      r[2] = bn;
      r[3] = qw;
      r[4] = qa;
      r[5] = na;
      r[6] = qb;
      r[7] = nb;
      r[16] = nw;
      r[17] = kernel;
      r[18] = p.q_row0 + row_end;
    }
    r[8 + wave] = n_act;
  }
#else
  (void)p, (void)slot, (void)kernel, (void)bh, (void)bm, (void)bn, (void)qw, (void)nw, (void)qa, (void)na, (void)qb,
      (void)nb, (void)wave, (void)lane, (void)n_act, (void)row_end;
#endif
}
__device__ __forceinline__ void record_tiles(const Params& p, int kernel, int bh, int bm, int bn, int qw, int nw, int qa,
                                             int na, int qb, int nb, int wave, int lane, int n_act, int row_end) {
  record_tiles_at(p, blockIdx.x, kernel, bh, bm, bn, qw, nw, qa, na, qb, nb, wave, lane, n_act, row_end);
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
    sg.q_base = b * p.stride_b_q + h * p.stride_h_q + (int64_t)p.q_row0 * p.stride_s;
    sg.kv_base = b * p.stride_b_k + h * p.stride_h_k + p.kv_start * p.stride_s;
    sg.lse_base = (int64_t)bh * p.lse_rows + p.q_row0;
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
  // (the last key visible to the workgroup's last real query: a ragged last tile streams no further)
  const int k_last = CAUSAL ? (int)max((int64_t)-1, min((int64_t)Nkv - 1, min(q_wg + T::BM, Nq) - 1 + delta)) : Nkv - 1;
  const int n_kt_a = k_last >= k_begin ? (k_last - k_begin) / T::BN + 1 : 0;
  // the light tile of a pair (PAIR: no window, every tile sees key 0)
  const int n_kt_b = qt_b >= 0 ? (int)min((int64_t)Nkv - 1, qt_b * T::BM + T::BM - 1 + delta) / T::BN + 1 : 0;
  const int n_kt = n_kt_a + n_kt_b;
  const int q_wg_a = q_wg;
  int n_act = 0;  // tiles this wave computes on (recorded by the test-only build)
  if (n_kt == 0) {  // no query of this workgroup sees any key of the chunk: O = 0, lse = -inf
    record_tiles(p, 0, bh, T::BM, T::BN, T::QW, T::NW, q_wg, 0, -1, 0, wave, lane, 0, p.Nq);
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
  // (16-byte stores: lanes 16 apart, the same row, exchange the pieces of two d tiles, as in fa_fwd_16pp)
  auto finish = [&]() __attribute__((always_inline)) {
    const bool odd = (g & 1) != 0;
#pragma unroll
    for (int qg = 0; qg < T::QG; ++qg) {
      const float l = wave_sum_xor16_32(l_part[qg]);
      const float inv = uacc[qg][0] > 0.0f ? 1.0f / uacc[qg][0] : 0.0f;
      const int qi = q0 + 16 * qg + li;
#pragma unroll
      for (int m = 0; m < T::DT / 2; ++m) {
        const f32x4_t o0 = oacc[qg][2 * m] * inv, o1 = oacc[qg][2 * m + 1] * inv;
        const uint32_t a0 = E::pack2(o0[0], o0[1]), a1 = E::pack2(o0[2], o0[3]);
        const uint32_t b0 = E::pack2(o1[0], o1[1]), b1 = E::pack2(o1[2], o1[3]);
        const uint32_t s0 = odd ? a0 : b0, s1 = odd ? a1 : b1;
        const uint32_t r0 = __shfl_xor(s0, 16), r1 = __shfl_xor(s1, 16);  // (the partner has the same row)
        const u32x4_t w = odd ? u32x4_t{r0, r1, b0, b1} : u32x4_t{a0, a1, r0, r1};
        const int col = odd ? 16 * (2 * m + 1) + 4 * (g - 1) : 16 * (2 * m) + 4 * g;
        if (qi < Nq) *(u32x4_t*)(og_ptr + qi * p.stride_s + col) = w;
      }
      if (g == 0 && qi < Nq) p.lse[sg.lse_base + qi] = (m_ref[qg] + __builtin_log2f(l)) * kLn2;
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
    // the wave's real queries see some key of this tile (causal: its first key is not after the last
    // query's position; window: its last key is not before the first query's window)
    const bool active = q0 < Nq && (!CAUSAL || key0 <= min(q0 + T::QW, Nq) - 1 + delta) &&
                        (!WINDOW || min(key0 + T::BN, Nkv) - 1 >= q0 + delta - window);
    if (active) {
      ++n_act;
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
          // a row that has seen no visible key yet takes a huge negative reference: its sums stay 0, and its
          // first visible key gives P = inf, which fails the limit check and moves the reference to the
          // row's real maximum (a finite placeholder such as 0 could leave every later P underflowing)
          float m_new = fmaxf(m_ref[qg], mx * cexp);
          if (m_new == kNegInf) m_new = kNoKeyRef;
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
  record_tiles(p, 0, bh, T::BM, T::BN, T::QW, T::NW, q_wg_a, n_kt_a, PAIR ? qt_b * T::BM : -1, n_kt_b, wave, lane,
               n_act, p.Nq);
}

// ------------------------------------------------------------------------------------------------
// 16-bit inputs, ping-pong schedule: 8 waves, whole problems without a window
// ------------------------------------------------------------------------------------------------
// Waves w and w + 4 share a SIMD.  Per K/V tile j every wave runs two phases:
//   matrix phase M(j): O^T += V^T P^T of tile j-1 (its V fragments already sit in registers) while the
//                      K fragments of tile j are read from LDS, then S^T = K Q^T of tile j;
//   vector phase V(j): the transposing reads of tile j's V fragments into registers, then the mask and
//                      the online softmax of S(j) into P(j).
// One workgroup barrier per tile: waves 0-3 pass it after their vector phases, waves 4-7 after their
// matrix phases, so between two barriers waves 0-3 run M(j) then V(j) while waves 4-7 run V(j-1) then
// M(j).  On every SIMD one wave issues MFMAs while the other computes exponentials, and within the
// interval the two may drift (the formula page, section "ops-transformer 中的实现", has the matrix and
// vector units of the Ascend core work side by side; here the two waves of a SIMD take those roles in
// turn).  The matrix wave runs at the higher issue priority.  K/V tiles stream through a 4-stage LDS
// ring: tile j+2 is issued early in M(j) (behind its first two products), once every wave has passed the
// barrier after its last use of tile j-2; the extra stage lets a vector phase end with its V reads still in
// flight (they are consumed by the next matrix phase).  A whole causal problem runs as pairs: a workgroup takes the heavy
// query tile n-1-r and then the light tile r of one head over one continuous K/V stream, so every
// workgroup computes n+1 tiles of 256 rows by 256 keys.
template <int D, bool IS_BF16, bool CAUSAL, bool PAIR, bool CHUNK = false>
__global__ __launch_bounds__(512, 1) void fa_fwd_16pp(Params p) {
  typedef Tile16<D, 8> T;
  typedef Elem<IS_BF16> E;
  typedef typename E::vec8 vec8;
  // four stages for K and four for V, eight LDS objects (a stage fixed at compile time lets the compiler
  // see that reads of one stage do not wait for the DMA filling another; as fields of one struct, which
  // would fix their order, they made it wait for every DMA in flight).  The compiler lays a kernel's
  // LDS objects out in name order: the V stages (lds_a*) take the low 64 KiB and the K stages (lds_b*) the
  // 64 KiB above.  A DS instruction's immediate offset has 16 bits, so the transposing V reads (two per
  // fragment, 8 base registers) address every stage with an immediate, and the K reads (one per fragment,
  // 4 base registers) do the same from bases that already hold the 64 KiB (kb below); with the V stages
  // above 64 KiB every V read had cost a VALU add, 32 per wave and tile.
  __shared__ __attribute__((aligned(1024))) uint8_t lds_a_v0[T::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_a_v1[T::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_a_v2[T::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_a_v3[T::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_b_k0[T::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_b_k1[T::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_b_k2[T::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_b_k3[T::TILE_BYTES];
  constexpr int K_HIGH = 4 * T::TILE_BYTES >= 65536 ? 65536 : 0;  // what kb holds of the K stages' address

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = wave >> 2;  // 0: waves 0-3, 1: waves 4-7 (one phase behind)
  const int g = lane >> 4;
  const int li = lane & 15;

  // PAIR: a chain of n_pairs heavy/light pairs of one head (group c of the head's pairs, r = (c + 1) n_pairs
  // - 1 down to c n_pairs; pair r is query tile n_full - 1 - r, then tile r).  The launcher pairs only whole
  // causal problems of an even number of full 256-row tiles and splits the pairs evenly.  Descending, the
  // only unit of four tiles (tile 0) ends its chain.
  // CHUNK (with PAIR): a key chunk split into row ranges (rows counted from q_row0).  Blocks [0, P8) run the
  // pairs of its square (rows 0 .. Nkv - 1, keys 0 .. Nkv - 1); blocks [P8, P8 + R8) run the rows
  // Nkv .. Nq - 1, which see every key, in chains of n_chain units of 256 rows (the pair code's masks leave
  // them alone: their rows lie past every key); the remaining blocks, the shortest, write O = 0 and
  // lse = -inf for the rows -n_empty .. -1, which see none, into the launch's tail.  P8 and R8 are the
  // block counts padded to multiples of 8, so each range starts on the first XCD.
  int bh, qt, c_grp = 0, n_pairs = 1, n_chain = 1;
  bool pair_wg = PAIR, zero_wg = false;
  const int n_full = (CHUNK ? p.Nkv : p.Nq) / T::BM;
  if constexpr (CHUNK) {
    const int heads = p.B * p.H;
    const int P8 = (p.n_units + 7) & ~7, R = p.n_rect / p.n_chain * heads, R8 = (R + 7) & ~7;
    int bid = blockIdx.x;
    if (bid < P8) {
      if (bid >= p.n_units) return;
      unit_of(bid, p.n_units, p.n_qtiles, false, bh, c_grp);
      n_pairs = (n_full / 2) / p.n_qtiles;
      qt = n_full - (c_grp + 1) * n_pairs;
    } else if (bid < P8 + R8) {
      bid -= P8;
      if (bid >= R) return;
      unit_of(bid, R, R / heads, false, bh, c_grp);
      n_chain = p.n_chain;
      qt = n_full + c_grp * n_chain;
      pair_wg = false;
    } else {
      bid -= P8 + R8;
      const int Z = (p.n_empty + T::BM - 1) / T::BM * heads;
      if (bid >= Z) return;
      unit_of(bid, Z, Z / heads, false, bh, qt);
      zero_wg = true;
    }
  } else if constexpr (PAIR) {
    unit_of(blockIdx.x, p.n_units, p.n_qtiles, false, bh, c_grp);
    n_pairs = (n_full / 2) / p.n_qtiles;
    qt = n_full - (c_grp + 1) * n_pairs;
  } else {
    unit_of(blockIdx.x, p.n_units, p.n_qtiles, CAUSAL, bh, qt);
  }
  // unit u of the chain: its query tile and its tile count (keys 0 .. the last key of its last row; a chunk's
  // rows after the square: consecutive tiles, every key)
  auto qt_of = [&](int u) __attribute__((always_inline)) {
    if (CHUNK && !pair_wg) return qt + u;
    const int r = (c_grp + 1) * n_pairs - 1 - (u >> 1);
    return (u & 1) ? r : n_full - 1 - r;
  };
  auto q0_of_unit = [&](int u) __attribute__((always_inline)) { return qt_of(u) * T::BM + wave * T::QW; };
  auto nt_of_unit = [&](int u) __attribute__((always_inline)) {
    return (CHUNK && !pair_wg) ? p.Nkv / T::BN : (qt_of(u) + 1) * (T::BM / T::BN);
  };
  const int n_chain_units = pair_wg ? 2 * n_pairs : n_chain;  // units this block runs
  const int b = bh / p.H, h = bh - (bh / p.H) * p.H;
  const SeqGeom sg = seq_geometry<CAUSAL, false>(p, b, h, bh);
  const int Nq = sg.Nq, Nkv = sg.Nkv;
  const int64_t delta = PAIR ? 0 : sg.delta;  // pairs: whole causal problems (queries and keys from 0)
  const int q0a = qt * T::BM + wave * T::QW;  // first query of this wave in the (first) unit

  const uint16_t* __restrict__ qg_ptr = (const uint16_t*)p.q + sg.q_base;
  const uint8_t* __restrict__ kg_ptr = (const uint8_t*)p.k + 2 * sg.kv_base;
  const uint8_t* __restrict__ vg_ptr = (const uint8_t*)p.v + 2 * sg.kv_base;
  uint16_t* og_ptr = (uint16_t*)p.o + sg.q_base;

  if (CHUNK && zero_wg) {  // rows -n_empty + 256 qt .. (at most) -1: no visible key
    const int r0 = -p.n_empty + qt * T::BM, r1 = min(r0 + T::BM, 0);
    constexpr int CPR = D / 8;  // 16-byte pieces per row
    for (int i = threadIdx.x; i < (r1 - r0) * CPR; i += 64 * T::NW)
      *(u32x4_t*)(og_ptr + (int64_t)(r0 + i / CPR) * p.stride_s + 8 * (i % CPR)) = u32x4_t{0u, 0u, 0u, 0u};
    for (int i = threadIdx.x; i < r1 - r0; i += 64 * T::NW) p.lse[sg.lse_base + r0 + i] = kNegInf;
    record_tiles(p, 1, bh, T::BM, T::BN, T::QW, T::NW, r0, 0, -1, 0, wave, lane, 0, r1);
    return;
  }

  // tiles of 64 keys from key 0 up to the last key visible to the unit's last query
  const int q_wg = qt * T::BM;
  // (the last key visible to the workgroup's last real query: a ragged last tile streams no further)
  const int k_last = CAUSAL ? (int)max((int64_t)-1, min((int64_t)Nkv - 1, min(q_wg + T::BM, Nq) - 1 + delta)) : Nkv - 1;
  const int n_kt_a = k_last >= 0 ? k_last / T::BN + 1 : 0;
  if (n_kt_a == 0) {  // no key at all (an empty chunk): O = 0, lse = -inf
#pragma unroll
    for (int qg = 0; qg < T::QG; ++qg) {
      const int qi = q0a + 16 * qg + li;
      if (qi < Nq) {
#pragma unroll
        for (int dt = 0; dt < T::DT; ++dt) *(u32x2_t*)(og_ptr + qi * p.stride_s + 16 * dt + 4 * g) = u32x2_t{0u, 0u};
        if (g == 0) p.lse[sg.lse_base + qi] = kNegInf;
      }
    }
    return;
  }

  // K/V tile DMA, as in fa_fwd_16: buffer loads straight into LDS, the swizzle applied on the global side
  const int row_bytes = (int)(2 * p.stride_s);
  const int span = (Nkv - 1) * row_bytes + T::ROW_BYTES;
  const __amdgpu_buffer_rsrc_t kbuf = __builtin_amdgcn_make_buffer_rsrc((void*)kg_ptr, 0, span, kBufferFlags);
  const __amdgpu_buffer_rsrc_t vbuf = __builtin_amdgcn_make_buffer_rsrc((void*)vg_ptr, 0, span, kBufferFlags);
  int voff_k, voff_v;
  {
    const int slot = wave * 64 + lane;
    const int row = slot / T::CHUNKS, pc = slot % T::CHUNKS;
    voff_k = row * row_bytes + ((pc ^ T::swz_k(row)) << 4);
    voff_v = row * row_bytes + ((pc ^ T::swz_v(row)) << 4);
  }
  const int load_step = (T::NW * 64 / T::CHUNKS) * row_bytes;
  auto kstage = [&](auto st) __attribute__((always_inline)) -> uint8_t* {
    constexpr int s = decltype(st)::value % 4;
    if constexpr (s == 0) return lds_b_k0;
    else if constexpr (s == 1) return lds_b_k1;
    else if constexpr (s == 2) return lds_b_k2;
    else return lds_b_k3;
  };
  auto vstage = [&](auto st) __attribute__((always_inline)) -> uint8_t* {
    constexpr int s = decltype(st)::value % 4;
    if constexpr (s == 0) return lds_a_v0;
    else if constexpr (s == 1) return lds_a_v1;
    else if constexpr (s == 2) return lds_a_v2;
    else return lds_a_v3;
  };
  auto issue_tile = [&](int key, uint8_t* kdst, uint8_t* vdst) __attribute__((always_inline)) {
    const int soff = key * row_bytes;
    // The LDS destination (m0) of every load is a stage's address plus this wave's offset.  Left visible,
    // the compiler keeps all 16 sums live in SGPRs; in the causal build they then spill to VGPR lanes,
    // and every DMA issue at the start of a matrix phase waits on v_readlane, a VALU instruction that
    // competes with the other wave's exponentials.  One SGPR and a scalar add per load instead.
    int wave_off = wave * 1024;
    asm volatile("" : "+s"(wave_off));
#pragma unroll
    for (int i = 0; i < T::LOADS; ++i) {
      const int lds_off = i * T::NW * 1024 + wave_off;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kbuf, (lds_void_t*)(kdst + lds_off), 16, voff_k, soff + i * load_step, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vbuf, (lds_void_t*)(vdst + lds_off), 16, voff_v, soff + i * load_step, 0, 0);
    }
  };
  constexpr int TILE_LOADS = 2 * T::LOADS;  // DMA instructions per wave and tile
  constexpr int Q_LOADS = T::QG * T::DC;    // global load instructions of one Q fragment set
  // store instructions of finish() that a wait may leave in flight: the O stores (16 bytes per lane, one
  // per two d tiles); the lse stores are not counted, which only makes the waits stricter
  constexpr int O_STORES = T::QG * T::DT / 2;

  // Q fragments; FLIP: apply the sign flip of a negative scale now (else flip_q() does it before the first
  // use: a flip right after a load made the compiler wait there for every load in flight, the DMA too)
  vec8 qf[T::QG][T::DC];
  auto load_q = [&](int qbase, auto flip_c) __attribute__((always_inline)) {
#pragma unroll
    for (int qg = 0; qg < T::QG; ++qg) {
      const int qrow = min(qbase + 16 * qg + li, Nq - 1);
#pragma unroll
      for (int c = 0; c < T::DC; ++c) {
        u32x4_t raw = *(const u32x4_t*)(qg_ptr + qrow * p.stride_s + 32 * c + 8 * g);
        if constexpr (decltype(flip_c)::value) raw ^= p.qsign;
        qf[qg][c] = __builtin_bit_cast(vec8, raw);
      }
    }
  };
  auto flip_q = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int qg = 0; qg < T::QG; ++qg)
#pragma unroll
      for (int c = 0; c < T::DC; ++c) qf[qg][c] = __builtin_bit_cast(vec8, __builtin_bit_cast(u32x4_t, qf[qg][c]) ^ p.qsign);
  };

  const float cexp = p.c;
  float m_ref[T::QG], l_part[T::QG];
  f32x4_t oacc[T::QG][T::DT], uacc[T::QG];
  auto reset = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int qg = 0; qg < T::QG; ++qg) {
      m_ref[qg] = kNegInf;
      l_part[qg] = 0.f;
      uacc[qg] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int dt = 0; dt < T::DT; ++dt) oacc[qg][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
  };
  reset();

  int kb[T::DC], vb[T::DT];
#pragma unroll
  for (int c = 0; c < T::DC; ++c) {
    kb[c] = K_HIGH + li * T::ROW_BYTES + (((4 * c + g) ^ T::swz_k(li)) << 4);
    asm volatile("" : "+v"(kb[c]));  // kept whole: the stage address minus K_HIGH becomes the immediate
  }
#pragma unroll
  for (int dt = 0; dt < T::DT; ++dt) {
    const int vrow = 4 * g + (li >> 2);
    const int col = 16 * dt + 4 * (li & 3);
    vb[dt] = vrow * T::ROW_BYTES + (((col >> 3) ^ T::swz_v(vrow)) << 4) + (col & 7) * 2;
  }

  // O = acc / u and lse of the unit's rows.  A lane holds 4 columns of a row per 16-wide d tile, so direct
  // stores would write 8 bytes per lane, 32 contiguous bytes per row and instruction.  Lanes g and g ^ 1
  // (16 lanes apart, the same row) exchange the pieces of two d tiles instead: even g then holds columns 32 m + 4 g ..
  // + 7, odd g columns 32 m + 16 + 4 (g - 1) .. + 7, and each 16-byte store writes 64 contiguous bytes of
  // 16 rows.  At a unit switch the narrow stores cost about 3 % of the kernel.
  auto finish = [&](int q0) __attribute__((always_inline)) {
    const bool odd = (g & 1) != 0;
#pragma unroll
    for (int qg = 0; qg < T::QG; ++qg) {
      const float l = wave_sum_xor16_32(l_part[qg]);
      const float inv = uacc[qg][0] > 0.0f ? 1.0f / uacc[qg][0] : 0.0f;
      const int qi = q0 + 16 * qg + li;
#pragma unroll
      for (int m = 0; m < T::DT / 2; ++m) {
        const f32x4_t o0 = oacc[qg][2 * m] * inv, o1 = oacc[qg][2 * m + 1] * inv;
        const uint32_t a0 = E::pack2(o0[0], o0[1]), a1 = E::pack2(o0[2], o0[3]);  // d tile 2m, own columns
        const uint32_t b0 = E::pack2(o1[0], o1[1]), b1 = E::pack2(o1[2], o1[3]);  // d tile 2m+1
        // even lanes keep tile 2m and send tile 2m+1; odd lanes the reverse
        const uint32_t s0 = odd ? a0 : b0, s1 = odd ? a1 : b1;
        const uint32_t r0 = __shfl_xor(s0, 16), r1 = __shfl_xor(s1, 16);  // the partner's (lane ^ 16) half
        const u32x4_t w = odd ? u32x4_t{r0, r1, b0, b1} : u32x4_t{a0, a1, r0, r1};
        const int col = odd ? 16 * (2 * m + 1) + 4 * (g - 1) : 16 * (2 * m) + 4 * g;
        // (pairs: every row is real, and every store must issue: the waits after a unit switch count them)
        if (PAIR || qi < Nq) *(u32x4_t*)(og_ptr + qi * p.stride_s + col) = w;
      }
      if (g == 0 && qi < Nq) p.lse[sg.lse_base + qi] = (m_ref[qg] + __builtin_log2f(l)) * kLn2;
    }
  };

  constexpr int NF = T::KC * T::DT;  // V^T fragments per tile (= K fragments per tile, KT * DC)
  static_assert(NF == T::KT * T::DC, "one K fragment read per V fragment product");
  // Every wave runs every tile of the workgroup's stream: on a tile wholly above its queries the mask
  // leaves P = 0, so the products add nothing, and the barrier waits for the busiest SIMD either way.
  constexpr int H = NF / 2;
  vec8 vfr[H];                   // first half of the previous tile's V^T fragments (read in its vector phase)
  uint32_t pf[T::QG][T::KC][4];  // P of the previous tile, B-operand layout
  f32x4_t s[T::QG][T::KT];       // S^T of the current tile

  // V^T fragment f of a tile (transposing reads): lanes 4e..4e+3 of each 16-lane group address row e
  // and lane li receives column li of those rows
  auto v_frag = [&](const uint8_t* vs, int f) __attribute__((always_inline)) {
    const int kc = f / T::DT, dt = f % T::DT;
    const uint8_t* a0 = vs + vb[dt] + 32 * kc * T::ROW_BYTES;
    const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)a0);
    const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(a0 + 16 * T::ROW_BYTES));
    u32x4_t w = {__builtin_bit_cast(u32x2_t, lo)[0], __builtin_bit_cast(u32x2_t, lo)[1],
                 __builtin_bit_cast(u32x2_t, hi)[0], __builtin_bit_cast(u32x2_t, hi)[1]};
    return __builtin_bit_cast(vec8, w);
  };
  // K fragment g = c * KT + kt of a tile (row reads), in the order the S^T products use them
  auto k_frag = [&](const uint8_t* ks, int g) __attribute__((always_inline)) {
    return *(const vec8*)(ks + (kb[g / T::KT] - K_HIGH) + 16 * (g % T::KT) * T::ROW_BYTES);
  };
  auto pv_mfma = [&](int f, const vec8& vf) __attribute__((always_inline)) {
    const int kc = f / T::DT, dt = f % T::DT;
#pragma unroll
    for (int qg = 0; qg < T::QG; ++qg) {
      u32x4_t w = {pf[qg][kc][0], pf[qg][kc][1], pf[qg][kc][2], pf[qg][kc][3]};
      oacc[qg][dt] = E::mfma(vf, __builtin_bit_cast(vec8, w), oacc[qg][dt]);
    }
  };
  // u += the all-ones product of P's key chunk kc (the rounded P summed per query)
  auto u_mfma = [&](int kc) __attribute__((always_inline)) {
#pragma unroll
    for (int qg = 0; qg < T::QG; ++qg) {
      u32x4_t w = {pf[qg][kc][0], pf[qg][kc][1], pf[qg][kc][2], pf[qg][kc][3]};
      uacc[qg] = E::mfma(E::ones(), __builtin_bit_cast(vec8, w), uacc[qg]);
    }
  };
  // O^T += V^T P^T of the previous tile (and u): the first half of its fragments is in registers, the
  // second half is read from LDS behind the first half's products.  Products into one accumulator are at
  // least 8 MFMAs apart (a dependent MFMA issued sooner waits for its predecessor's result).
  auto pv_first = [&](const uint8_t* vs_prev, vec8 (&v2)[H]) __attribute__((always_inline)) {
    u_mfma(0);
#pragma unroll
    for (int f = 0; f < H; ++f) {
      pv_mfma(f, vfr[f]);
      v2[f] = v_frag(vs_prev, H + f);
      if (f == H / 2 && T::KC > 1) u_mfma(1);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Every wave issues tile j+2's DMA in its matrix phase M(j), behind the phase's first two products (past
  // the stream's end it fetches the last tile again into the free stage; issued first, the DMA held up the
  // first products: C3 +1.5 %, C5 +1.8 % from the move) and, right before its barrier (after V(j) for waves
  // 0-3, after M(j) for waves 4-7), waits until its share of tile j+1 has landed: at most tile j+2's loads
  // (and the Q loads issued after them) stay in flight, a constant count.  Stage safety: tile j+2 refills
  // the stage of tile j-2, whose last readers (waves 4-7's M(j-1), which drains its LDS reads) finish
  // before the barrier that precedes any wave's M(j); tile j+1 is first read after the next barrier.
  // (jl counts the unit's tiles; every unit starts at key 0, in stage 0)
  auto issue_next = [&](int jl, auto st, int nt, bool more) __attribute__((always_inline)) {
    constexpr int S = decltype(st)::value;
    const int jn = jl + 2;
    const int key = (jn < nt ? jn : (more ? jn - nt : nt - 1)) * T::BN;
    issue_tile(key, kstage(std::integral_constant<int, S + 2>()), vstage(std::integral_constant<int, S + 2>()));
  };

  // matrix phase M(j): P.V of tile j-1 (stage st-1), then S of tile j (stage st).  PV: there is a tile
  // j-1 (not on the kernel's first tile, where stage st-1 holds no data yet).  qload: the last tile of a
  // unit that another follows, after whose S^T the next unit's Q (first row q0_next) is loaded
  // flip: the unit's first tile, whose Q was loaded unflipped
  // stores: a unit's output was stored after the DMA of the tile this barrier waits for (the stores may
  // stay in flight: vmcnt retires in issue order, so the count still covers that tile)
  auto mphase = [&](int jl, auto st, auto pv_c, bool qload, int nt, bool more, int q0_next, bool flip = false,
                    bool stores = false) __attribute__((always_inline)) {
    constexpr int S = decltype(st)::value;
    constexpr bool PV = decltype(pv_c)::value;
    __builtin_amdgcn_s_setprio(1);
    const uint8_t* ks = kstage(st);
    vec8 ka[H], kc2[H];
    if constexpr (PV) {
      vec8 v2[H];
      // (pv_first with the DMA issued behind the first two products)
#pragma unroll
      for (int f = 0; f < H; ++f) {
        pv_mfma(f, vfr[f]);
        v2[f] = v_frag(vstage(std::integral_constant<int, S + 3>()), H + f);
        if (f == 0) u_mfma(0);
        if (f == 1) issue_next(jl, st, nt, more);
        if (f == H / 2 && T::KC > 1) u_mfma(1);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int f = 0; f < H; ++f) {
        pv_mfma(H + f, v2[f]);
        ka[f] = k_frag(ks, f);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      issue_next(jl, st, nt, more);
#pragma unroll
      for (int f = 0; f < H; ++f) ka[f] = k_frag(ks, f);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (flip) flip_q();
    // S^T = K Q^T, d-chunk outer (products into one accumulator KT * QG MFMAs apart); the first half of
    // the d-chunks runs while the second half's fragments are read
#pragma unroll
    for (int kt = 0; kt < T::KT; ++kt)
#pragma unroll
      for (int qg = 0; qg < T::QG; ++qg) s[qg][kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < T::DC; ++c)
#pragma unroll
      for (int kt = 0; kt < T::KT; ++kt) {
        const int g = c * T::KT + kt;
        const vec8 kf = g < H ? ka[g] : kc2[g - H];
#pragma unroll
        for (int qg = 0; qg < T::QG; ++qg) s[qg][kt] = E::mfma(kf, qf[qg][c], s[qg][kt]);
        if (g < H) kc2[g] = k_frag(ks, H + g);
        __builtin_amdgcn_sched_barrier(0);
      }
    if (qload) load_q(q0_next, std::false_type());
    __builtin_amdgcn_s_setprio(0);
    if (grp == 1) {  // group 1's barrier closes its matrix phase
      if (qload) __builtin_amdgcn_s_waitcnt(waitcnt_vm(TILE_LOADS + Q_LOADS));
      else if (stores) __builtin_amdgcn_s_waitcnt(waitcnt_vm(TILE_LOADS + O_STORES));
      else __builtin_amdgcn_s_waitcnt(waitcnt_vm(TILE_LOADS));
      __builtin_amdgcn_sched_barrier(0);
      lds_barrier();
    }
  };

  // vector phase V(j); FIRST: the unit's first tile, which sets the reference maximum (every wave sees
  // key 0 of a whole causal or non-causal problem)
  // (first_rt: the same as FIRST, decided at run time)
  auto vphase = [&](int jl, auto st, auto first_c, bool qload, int q0, bool first_rt = false, bool stores = false)
                    __attribute__((always_inline)) {
    constexpr bool FIRST = decltype(first_c)::value;
    const int key0 = jl * T::BN;
    // (pairs: no ragged tile, and the causal edge in 32 bits)
    const bool need_mask = PAIR ? key0 + T::BN - 1 > q0
                                : (CAUSAL && key0 + T::BN - 1 > q0 + delta) || (key0 + T::BN > Nkv);
    if (need_mask) {
      keep_branch();
      const int dq0 = PAIR ? max(-512, min(512, q0 - key0))
                           : CAUSAL ? (int)max((int64_t)-512, min((int64_t)512, q0 + delta - key0)) : 0;
      const int kend = PAIR ? 512 : min(512, Nkv - key0);
#pragma unroll
      for (int qg = 0; qg < T::QG; ++qg) {
        const int hi = (CAUSAL ? min(kend - 1, dq0 + 16 * qg + li) : kend - 1) - 4 * g;
#pragma unroll
        for (int kt = 0; kt < T::KT; ++kt) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (16 * kt + r > hi) s[qg][kt][r] = kNegInf;
          // each compare's lane mask (an SGPR pair) dies at its select: hoisted together, the 32 compares
          // of a tile held 64 SGPRs and spilled
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    float part[T::QG];
    auto expo = [&](int qg) __attribute__((always_inline)) {
      const float neg_m = -m_ref[qg];
      float acc = 0.f;
#pragma unroll
      for (int kt = 0; kt < T::KT; ++kt) {
        float pv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) pv[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qg][kt][r], cexp, neg_m));
        const float t4 = (pv[0] + pv[1]) + (pv[2] + pv[3]);
        acc = kt == 0 ? t4 : acc + t4;  // (0 + x is not folded: it would turn -0 into +0)
        const int kc = kt >> 1, half = kt & 1;
        pf[qg][kc][2 * half + 0] = E::pack2(pv[0], pv[1]);
        pf[qg][kc][2 * half + 1] = E::pack2(pv[2], pv[3]);
      }
      part[qg] = acc;
    };
    bool slow[T::QG];
#pragma unroll
    for (int qg = 0; qg < T::QG; ++qg) {
      if (FIRST || first_rt) {
        slow[qg] = true;
      } else {
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
        float m_new = fmaxf(m_ref[qg], mx * cexp);
        if (m_new == kNegInf) m_new = kNoKeyRef;  // no visible key yet (as in fa_fwd_16)
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
    __builtin_amdgcn_sched_barrier(0);
    // the first half of this tile's V^T fragments, for the next matrix phase
    const uint8_t* vs = vstage(st);
#pragma unroll
    for (int f = 0; f < H; ++f) vfr[f] = v_frag(vs, f);
    // no LDS wait: the V reads may still be in flight (the next matrix phase consumes them, a barrier
    // before the DMA refills this stage)
    __builtin_amdgcn_sched_barrier(0);
    if (grp == 0) {  // group 0's barrier closes its vector phase
      if (qload) __builtin_amdgcn_s_waitcnt(waitcnt_vm(TILE_LOADS + Q_LOADS));
      else if (stores) __builtin_amdgcn_s_waitcnt(waitcnt_vm(TILE_LOADS + O_STORES));
      else __builtin_amdgcn_s_waitcnt(waitcnt_vm(TILE_LOADS));
      compiler_fence();
      __builtin_amdgcn_s_barrier();
      compiler_fence();
    }
  };

  // Q before the first tiles: the wait for tile 0 covers it and leaves tile 1 in flight
  load_q(q0a, std::false_type());
  issue_tile(0, lds_b_k0, lds_a_v0);
  issue_tile(T::BN, lds_b_k1, lds_a_v1);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(TILE_LOADS));
  lds_barrier();

  const std::integral_constant<int, 0> st0;
  const std::integral_constant<int, 1> st1;
  const std::integral_constant<int, 2> st2;
  const std::integral_constant<int, 3> st3;
  const std::true_type first_c, pv_c;
  const std::false_type later_c;
  // The chain's units run in groups of four tiles (every unit's tile count is a multiple of 4: the launcher
  // runs this kernel only for causal pairs of whole 256-query tiles and for non-causal calls whose key
  // count is a multiple of 256), so every unit starts in stage 0.  One loop over the groups: a unit's
  // first matrix phase ends the previous unit, whose output is then stored, and its first vector phase
  // sets the reference maximum (a loop per unit nested in a loop over units spilled registers).
  int u = 0, nt = PAIR ? nt_of_unit(0) : n_kt_a, q0 = q0a;
  bool more = PAIR && n_chain_units > 1;
  int q0_next = more ? q0_of_unit(1) : q0;
  // the first group: its first matrix phase has no P.V
  mphase(0, st0, later_c, false, nt, more, q0_next, true);
  vphase(0, st0, first_c, false, q0);
  mphase(1, st1, pv_c, false, nt, more, q0_next);
  vphase(1, st1, later_c, false, q0);
  mphase(2, st2, pv_c, false, nt, more, q0_next);
  vphase(2, st2, later_c, false, q0);
  {
    const bool ql = nt == 4 && more;
    mphase(3, st3, pv_c, ql, nt, more, q0_next);
    vphase(3, st3, later_c, ql, q0);
  }
  int jl = 4;
#pragma unroll 1
  while (true) {
    bool unit_start = false;
    int q0_prev = q0;
    if (jl == nt) {
      if (!more) break;
      ++u;
      nt = nt_of_unit(u);
      q0 = q0_next;
      more = u + 1 < n_chain_units;
      q0_next = more ? q0_of_unit(u + 1) : q0;
      jl = 0;
      unit_start = true;
    }
    mphase(jl, st0, pv_c, false, nt, more, q0_next, unit_start);
    if (unit_start) {
      finish(q0_prev);
      reset();
    }
    // the two barriers after the previous unit's stores, in each group, leave them in flight
    vphase(jl, st0, later_c, false, q0, unit_start, unit_start);
    mphase(jl + 1, st1, pv_c, false, nt, more, q0_next, false, unit_start);
    vphase(jl + 1, st1, later_c, false, q0, false, unit_start);
    mphase(jl + 2, st2, pv_c, false, nt, more, q0_next);
    vphase(jl + 2, st2, later_c, false, q0);
    // the unit's last group loads the next unit's Q after its last S^T
    const bool ql = jl + 4 == nt && more;
    mphase(jl + 3, st3, pv_c, ql, nt, more, q0_next);
    vphase(jl + 3, st3, later_c, ql, q0);
    jl += 4;
  }
  const int q0_last = q0;
  // the last tile's P.V product (the second half of its V fragments from its stage, the last one)
  __builtin_amdgcn_s_setprio(1);
  {
    vec8 v2[H];
    pv_first(vstage(st3), v2);
#pragma unroll
    for (int f = 0; f < H; ++f) pv_mfma(H + f, v2[f]);
  }
  __builtin_amdgcn_s_setprio(0);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // the refetches past the end land before the LDS is released
  finish(q0_last);
  // every wave computes on every tile of the stream
  if (CHUNK && !pair_wg) {  // one record per unit of the chain, in slots past the grid's
    for (int i = 0; i < n_chain; ++i)
      record_tiles_at(p, gridDim.x + (blockIdx.x * n_chain + i), 1, bh, T::BM, T::BN, T::QW, T::NW,
                      qt_of(i) * T::BM, n_kt_a, -1, 0, wave, lane, n_kt_a, p.Nq);
  } else if (pair_wg) {
    for (int i = 0; i < n_pairs; ++i) {
      const int na = nt_of_unit(2 * i), nb = nt_of_unit(2 * i + 1);
      record_tiles_at(p, blockIdx.x * n_pairs + i, 1, bh, T::BM, T::BN, T::QW, T::NW, qt_of(2 * i) * T::BM, na,
                      qt_of(2 * i + 1) * T::BM, nb, wave, lane, na + nb, p.Nq);
    }
  } else {
    record_tiles(p, 1, bh, T::BM, T::BN, T::QW, T::NW, q_wg, n_kt_a, -1, 0, wave, lane, n_kt_a, p.Nq);
  }
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
  // (the last key visible to the workgroup's last real query: a ragged last tile streams no further)
  const int k_last = CAUSAL ? (int)max((int64_t)-1, min((int64_t)Nkv - 1, min(q_wg + T::BM, Nq) - 1 + delta)) : Nkv - 1;
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
    const bool active = q0 < Nq && (!CAUSAL || key0 <= min(q0 + T::QW, Nq) - 1 + delta) &&
                        (!WINDOW || min(key0 + T::BN, Nkv) - 1 >= q0 + delta - window);
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

template <int D, bool IS_BF16, bool CAUSAL, bool PAIR>
static hipError_t launch16pp(Params p, hipStream_t stream) {
  typedef Tile16<D, 8> T;
  p.n_qtiles = (p.Nq + T::BM - 1) / T::BM;
  // Pairs: one heavy/light pair per workgroup.  The kernel also takes chains of several pairs of a head
  // (n_qtiles = chains per head), which pay the prologue, the drain and the dispatch gap once; they
  // measured slower (C3: 2, 4, 8 pairs -0.5, -3, -11 %; C5 4 pairs -2 %): fewer workgroups of a head
  // stream its K/V side by side through L2.
  if (PAIR) p.n_qtiles = p.n_qtiles / 2;
  p.n_units = p.n_qtiles * p.B * p.H;
  hipLaunchKernelGGL((fa_fwd_16pp<D, IS_BF16, CAUSAL, PAIR>), dim3(p.n_units), dim3(512), 0, stream, p);
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

// A causal call whose key chunk starts at query row i0 = -delta >= 0 (the chunk's first key sits at that
// row's position) splits into three row ranges: rows 0 .. i0 - 1 see none of its keys, rows i0 .. i0 + Nkv - 1
// see it as a whole causal problem (row i0 + r sees keys 0 .. r), and every later row sees all of it.  One
// launch of the ping-pong kernel covers all three (CHUNK): the square's heavy/light pairs first, then the
// later rows as units of 256 rows, then blocks that write O = 0 and lse = -inf for the first rows.  Needs
// Nkv a multiple of 512 (pairs of 256-row tiles) and the rows after the square a multiple of 256.  (Three
// launches, one per range, measured no faster than fa_fwd_16 over the whole chunk: each paid its own
// ramp and tail, and a square of two pairs per head fills the GPU only twice over.)
#ifndef FA_CHUNK_CHAIN
#define FA_CHUNK_CHAIN 2
#endif
constexpr int kChunkChain = FA_CHUNK_CHAIN;

template <int D, bool IS_BF16>
static hipError_t launch16_chunk_split(Params p, int i0, hipStream_t stream) {
  typedef Tile16<D, 8> T;
  const int heads = p.B * p.H;
  const int rest = p.Nq - i0 - p.Nkv;
  p.q_row0 += i0;  // rows from the square's first row on
  p.Nq = p.Nkv + rest;
  p.delta = 0;
  p.n_qtiles = p.Nkv / (2 * T::BM);  // pairs per head (one pair per block)
  p.n_units = p.n_qtiles * heads;
  p.n_rect = rest / T::BM;
  p.n_empty = i0;
  // the rows after the square run in chains of up to kChunkChain units per block (the chain streams its
  // units' tiles back to back, as a pair does, so a block's start-up and drain are paid once per chain)
  p.n_chain = kChunkChain;
  while (p.n_chain > 1 && p.n_rect % p.n_chain != 0) p.n_chain /= 2;
  const int nz = (i0 + T::BM - 1) / T::BM;
  const int grid = ((p.n_units + 7) & ~7) + ((p.n_rect / p.n_chain * heads + 7) & ~7) + ((nz * heads + 7) & ~7);
  hipLaunchKernelGGL((fa_fwd_16pp<D, IS_BF16, true, true, true>), dim3(grid), dim3(512), 0, stream, p);
  return hipGetLastError();
}

template <int D, bool IS_BF16>
static hipError_t launch16_d(const Params& p, bool causal, hipStream_t stream) {
  // The ping-pong kernel runs non-causal calls whose query and key counts are multiples of 256 (its tiles
  // go in groups of four 64-key tiles, and every wave of a 256-query workgroup then has rows) and whole
  // causal problems of an even number of 256-query tiles, as heavy and light pairs, and the square and the
  // rows after it of a key chunk that splits into row ranges (launch16_chunk_split).  Windows, other
  // offsets and chunks keep fa_fwd_16 (with the mask on both edges of a window, or a chunk's diagonal cut
  // through 256-row units, the ping-pong kernel measured slower: many of their tiles are masked).
#ifndef FA_NO_PINGPONG
  constexpr bool kPingPong = true;
#else
  constexpr bool kPingPong = false;
#endif
  if (!causal) {
    if (kPingPong && p.Nq % 256 == 0 && p.Nkv > 0 && p.Nkv % 256 == 0) return launch16pp<D, IS_BF16, false, false>(p, stream);
    return launch16<D, IS_BF16, false, false>(p, stream);
  }
  if (p.window >= 0) return launch16<D, IS_BF16, true, true>(p, stream);
  // The whole causal problem (every query tile sees key 0): pairs of heavy and light tiles.  The pair
  // loop needs an even number of query tiles, each visiting an even number of 64-key tiles: the full
  // tiles do (BM is a multiple of 128), the last one does when the key count rounds up to an even
  // number of key tiles.  Pairs of 256-query tiles (8 waves) first, then of 128-query tiles.
  const bool whole = p.delta == 0 && p.Nq == p.Nkv && p.kv_start == 0;
  const bool even_keys = ((p.Nq + Tile16<D>::BN - 1) / Tile16<D>::BN) % 2 == 0;
  const auto pairs = [&](int bm) { return whole && even_keys && ((p.Nq + bm - 1) / bm) % 2 == 0; };
  // Pairs of 256-query tiles whose length is a multiple of 256 (every unit a whole number of groups of
  // four 64-key tiles) run the ping-pong kernel.
  if (kPingPong && pairs(Tile16<D, 8>::BM) && p.Nq % 256 == 0) return launch16pp<D, IS_BF16, true, true>(p, stream);
  if (pairs(Tile16<D, 8>::BM)) return launch16<D, IS_BF16, true, false, false, true, 8>(p, stream);
  if (pairs(Tile16<D, 4>::BM)) return launch16<D, IS_BF16, true, false, false, true, 4>(p, stream);
  // a key chunk (or keys starting at a later query's position) that splits into the three row ranges
  if (kPingPong && p.delta <= 0 && p.Nkv > 0 && p.Nkv % 512 == 0) {
    const int64_t rest = (int64_t)p.Nq + p.delta - p.Nkv;
    if (rest >= 0 && rest % 256 == 0) return launch16_chunk_split<D, IS_BF16>(p, (int)-p.delta, stream);
  }
  return launch16<D, IS_BF16, true, false>(p, stream);
}

template <int D>
static hipError_t launch32_d(const Params& p, bool causal, hipStream_t stream) {
  if (!causal) return launch32<D, false, false>(p, stream);
  return p.window >= 0 ? launch32<D, true, true>(p, stream) : launch32<D, true, false>(p, stream);
}

// A window is only used with causal attention (the entry point rejects it otherwise).
hipError_t launch(const Params& p_in, int dtype, int d, bool causal, hipStream_t stream) {
  Params p = p_in;
  if (p.lse_rows == 0) p.lse_rows = p.Nq;
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

#ifdef FA_TILE_COUNT
// Test-only entry point of libfa_tilecount.so: the device buffer (cap records of kTileRecInts ints) that the
// forward kernels launched after this call fill; null stops the recording.
extern "C" __attribute__((visibility("default"))) int fa_test_set_tile_record(int* buf, long long cap) {
  if (hipMemcpyToSymbol(HIP_SYMBOL(fa::g_tile_rec), &buf, sizeof(buf)) != hipSuccess) return 1;
  if (hipMemcpyToSymbol(HIP_SYMBOL(fa::g_tile_rec_cap), &cap, sizeof(cap)) != hipSuccess) return 1;
  return 0;
}
#endif
