// fa_bwd.hip -- attention backward kernels for gfx950 (MI355X, CDNA4), 16-bit inputs (fp32: fa_bwd32.hip).
//
// What is computed: for O = softmax(scale * Q K^T [+ causal mask]) V and an upstream gradient dO, the
// gradients dQ, dK, dV (the vector-Jacobian product).  With P the softmax probabilities,
//     dV = P^T dO,   dP = dO V^T,   D_i = sum_d dO_id O_id,   dS = P o (dP - D),
//     dQ = scale * dS K,   dK = scale * dS^T Q.
// P is never stored: it is recomputed tile by tile from the forward's per-row lse as
// exp(scale * q.k - lse).  Pages: ai6s.net/6a0d3bfb..., section "FlashAttention在昇腾NPU上怎么跑？",
// item 3 (the backward recomputes the forward's intermediates instead of storing the N x N matrices);
// hwcomputing.csdn.net/6a0d4681..., section "反向传播的特殊处理" (a deterministic mode next to one that
// accumulates with atomics).  D_i = rowsum(dO o O) equals sum_j P_ij dP_ij because O_i = sum_j P_ij v_j.
//
// Deterministic by construction: no atomics.  Two kernels, run in this order on one stream:
//   fa_bwd_dq   one workgroup per (b, h, 128-query tile); walks the K/V tiles (keys up to the tile's
//               last query when causal).  Computes D for its rows (stored to the caller's workspace),
//               then per K/V tile S^T = K Q^T, dP^T = V dO^T, dS^T, and dQ^T += K^T dS^T.
//   fa_bwd_dkdv one workgroup per (b, h, 128-key tile): 8 waves of 16 keys, two waves per SIMD; K and V
//               stay in registers; walks the 64-query Q/dO tiles (from the tile's first key on when
//               causal) with their rows' lse and D staged in LDS next to them.  Per 32-query step
//               S = Q K^T, dP = dO V^T, P, dS, then dV^T += dO^T P and dK^T += Q^T dS.
//
// gfx950 mapping (both kernels): v_mfma_f32_16x16x32_{bf16,f16}; the streamed operand arrives by
// buffer_load ... lds into a 2-stage LDS ring.  A tensor read both as rows (ds_read_b128, 16 consecutive
// rows at one logical 16-byte chunk) and transposed (ds_read_b64_tr_b16, 4 consecutive rows x 2 adjacent
// chunks) uses one XOR swizzle of the chunk index that keeps both access patterns free of bank conflicts.
// MFMA accumulator tiles are reused as the next product's operands without leaving registers: a 16x16
// C tile holds column j in lane j, which is the lane layout of both A rows and B columns.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <type_traits>

#include "fa_device.h"
#include "fa_bwd_launch.h"

namespace fa {
namespace {

constexpr float kLog2e = 1.44269504088896341f;
constexpr float kPosInf = __builtin_inff();
// dK/dV workgroup: waves, keys per wave (their product is 128, the tile of the launch grid), and the
// workgroups per CU the register budget is sized for
constexpr int kDkdvWaves = 8, kDkdvKeys = 16, kDkdvMinBlocks = 1;

template <int D>
struct BwdTile {
  static constexpr int NW = 4;            // waves per workgroup
  static constexpr int ROW_BYTES = D * 2;
  static constexpr int CHUNKS = D / 8;    // 16-byte chunks per row
  static constexpr int DC = D / 32;       // 32-wide d chunks: k dimension of the S and dP products
  static constexpr int DT = D / 16;       // 16-wide d tiles: rows of dQ^T, dK^T, dV^T
  // Chunk swizzle for tiles read both ways: row reads (ds_read_b128, lane group g reading rows r..r+15 at
  // one logical chunk) and transposing reads (ds_read_b64_tr_b16, rows 4e..4e+3 at logical chunks 2t,
  // 2t+1).  Chosen by measurement on gfx950 (SQ_LDS_BANK_CONFLICT of both access patterns over a 64-row
  // tile, for several candidates): these two are the simplest that are conflict-free for both patterns.
  // They depend on the row only through its low 3 bits, so 8-, 16- and 32-row steps keep a lane's offset.
  __device__ static __forceinline__ int swz(int row) { return D == 128 ? (row & 7) << 1 : row & 7; }
};

// 8 consecutive elements of a row held in LDS (row read): base + lane offset + row step.
template <typename vec8>
__device__ __forceinline__ vec8 row_frag(const uint8_t* base, int lane_off, int step) {
  return *(const vec8*)(base + lane_off + step);
}

// Transposing read of a 32-row x 16-column block: lane li of group g receives column li of rows
// 4g..4g+3 and 16+4g..16+4g+3 (relative to `step`), the A-operand layout of a product whose k index runs
// over those rows.
template <int ROW_BYTES, typename vec8>
__device__ __forceinline__ vec8 tr_frag(const uint8_t* base, int lane_off, int step) {
  const uint8_t* a0 = base + lane_off + step;
  const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)a0);
  const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(a0 + 16 * ROW_BYTES));
  u32x4_t w = {__builtin_bit_cast(u32x2_t, lo)[0], __builtin_bit_cast(u32x2_t, lo)[1],
               __builtin_bit_cast(u32x2_t, hi)[0], __builtin_bit_cast(u32x2_t, hi)[1]};
  return __builtin_bit_cast(vec8, w);
}

template <typename vec8>
__device__ __forceinline__ vec8 as_vec8(const uint32_t (&w)[4]) {
  return __builtin_bit_cast(vec8, u32x4_t{w[0], w[1], w[2], w[3]});
}

template <bool IS_BF16>
__device__ __forceinline__ float to_f32(typename Elem<IS_BF16>::vec8 x, int e) {
  return (float)x[e];
}

// Per-lane LDS offset of the transposing read of d tile dt: column 16*dt + 4*(li&3) of row 4g + (li>>2).
template <int D>
__device__ __forceinline__ int tr_offset(int li, int g, int dt) {
  typedef BwdTile<D> T;
  const int row = 4 * g + (li >> 2);
  const int col = 16 * dt + 4 * (li & 3);
  return row * T::ROW_BYTES + (((col >> 3) ^ T::swz(row)) << 4) + (col & 7) * 2;
}

// Per-lane LDS offsets: row reads of logical chunk 4c+g of row li, and the transposing reads of every d tile.
template <int D>
__device__ __forceinline__ void lane_offsets(int li, int g, int (&rb)[BwdTile<D>::DC], int (&tb)[BwdTile<D>::DT]) {
  typedef BwdTile<D> T;
#pragma unroll
  for (int c = 0; c < T::DC; ++c) rb[c] = li * T::ROW_BYTES + (((4 * c + g) ^ T::swz(li)) << 4);
#pragma unroll
  for (int dt = 0; dt < T::DT; ++dt) tb[dt] = tr_offset<D>(li, g, dt);
}

// Where one workgroup's (b, h) rows lie: the query and key counts, the key chunk, the query offset and
// window, the element offsets of the rows in Q/O/dO/dQ and K/V/dK/dV, and the index of the first row's lse
// and D.  For packed variable-length batches these come from sequence b's offsets (the two ends aligned
// under causal); offsets outside [0, total] or decreasing leave the sequence untouched (skip).
struct BwdGeom {
  int Nq, Nk, kv0, kv1;
  int64_t qoff, window, qhead, khead, row0;
  bool skip;
};

template <bool VARLEN, bool CAUSAL>
__device__ __forceinline__ BwdGeom bwd_geometry(const BwdParams& p, int b, int h, int bh) {
  BwdGeom gm;
  if constexpr (VARLEN) {
    const int qs = p.cu_q[b], qe = p.cu_q[b + 1], ks = p.cu_k[b], ke = p.cu_k[b + 1];
    gm.skip = qs < 0 || qe < qs || qe > p.total_q || ks < 0 || ke < ks || ke > p.total_k;
    gm.Nq = qe - qs;
    gm.Nk = ke - ks;
    gm.kv0 = 0;
    gm.kv1 = gm.Nk;
    gm.qoff = CAUSAL ? (int64_t)gm.Nk - gm.Nq : 0;
    gm.window = -1;
    gm.qhead = (int64_t)qs * p.stride_s + h * p.stride_h_q;
    gm.khead = (int64_t)ks * p.stride_s + h * p.stride_h_k;
    gm.row0 = (int64_t)h * p.total_q + qs;
  } else {
    gm.skip = false;
    gm.Nq = p.Nq;
    gm.Nk = p.Nk;
    gm.kv0 = p.kv_start;
    gm.kv1 = p.kv_start + p.kv_len;
    gm.qoff = p.q_offset;
    gm.window = p.window;
    gm.qhead = b * p.stride_b_q + h * p.stride_h_q;
    gm.khead = b * p.stride_b_k + h * p.stride_h_k;
    gm.row0 = (int64_t)bh * p.Nq;
  }
  return gm;
}

// ------------------------------------------------------------------------------------------------
// dQ (and D) : one workgroup per (b, h, 128-query tile)
// ------------------------------------------------------------------------------------------------
// PAIR (whole causal problems with an even number of 128-query tiles): workgroup r runs the heavy tile
// n-1-r and then the light tile r of one head over one continuous K/V stream, so every workgroup has the
// same work; the heavy tile's last step prefetches the light tile's first K/V tile and loads its Q and dO
// once its own S^T and dP^T products are done.
template <int D, bool IS_BF16, bool CAUSAL, bool WINDOW, bool VARLEN, bool PAIR = false>
__global__ __launch_bounds__(256, 2) void fa_bwd_dq(BwdParams p) {
  typedef BwdTile<D> T;
  typedef Elem<IS_BF16> E;
  typedef typename E::vec8 vec8;
  constexpr int NW = T::NW, QW = 32, BM = NW * QW, BN = 64;
  constexpr int QG = QW / 16, KT = BN / 16, KC = BN / 32;
  constexpr int TILE_BYTES = BN * T::ROW_BYTES;
  constexpr int LOADS = TILE_BYTES / (16 * 64 * NW);
  __shared__ __attribute__((aligned(1024))) uint8_t ks0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t ks1[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t vs0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t vs1[TILE_BYTES];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, li = lane & 15;
  static_assert(!PAIR || (CAUSAL && !WINDOW && !VARLEN), "pairs are for whole causal problems");
  int bh, qt, qt_b = -1;
  if constexpr (VARLEN) {
    unit_of_spread(blockIdx.x, p.n_tiles_q, CAUSAL, bh, qt);
    if (bh >= p.B * p.H) return;  // padding head of the grid
  } else if constexpr (PAIR) {
    int r;  // pair r of a head: tiles n-1-r and r (n_tiles_q counts pairs)
    unit_of(blockIdx.x, p.n_units_q, p.n_tiles_q, false, bh, r);
    qt = 2 * p.n_tiles_q - 1 - r;
    qt_b = r;
  } else {
    unit_of(blockIdx.x, p.n_units_q, p.n_tiles_q, CAUSAL, bh, qt);
  }
  const int b = bh / p.H, h = bh - (bh / p.H) * p.H;
  const BwdGeom gm = bwd_geometry<VARLEN, CAUSAL>(p, b, h, bh);
  if (VARLEN && (gm.skip || qt * BM >= gm.Nq)) return;  // a bad sequence, or a tile past its end
  const int Nq = gm.Nq, Nk = gm.Nk;
  const int64_t qoff = gm.qoff, window = gm.window;
  const int kv0 = gm.kv0, kv1 = gm.kv1;  // the key chunk [kv0, kv1)
  int q_wg = qt * BM, q0 = q_wg + wave * QW;  // (the light tile's, after a pair's switch)
  const int64_t qhead = gm.qhead, khead = gm.khead;
  const int64_t ss = p.stride_s;

  // K/V tiles from k_lo: the chunk's keys that some query of this workgroup sees
  const int k_lo = WINDOW ? (int)max((int64_t)kv0, q_wg + qoff - window) : kv0;
  const int k_hi = CAUSAL ? (int)min((int64_t)kv1 - 1, q_wg + BM - 1 + qoff) : kv1 - 1;
  const int n_kt_a = k_hi >= k_lo ? (k_hi - k_lo) / BN + 1 : 0;
  // a pair's light tile streams from key 0 to its own last query
  const int n_kt_b = PAIR ? (int)min((int64_t)kv1 - 1, (int64_t)qt_b * BM + BM - 1) / BN + 1 : 0;
  const int n_kt = n_kt_a + n_kt_b;
  // tile j of the stream: the first tile's, then the light tile's
  auto tile_of = [&](int j) __attribute__((always_inline)) { return PAIR && j >= n_kt_a ? j - n_kt_a : j; };
  // positions in 32 bits: the workgroup's first query position minus k_lo (and minus the window),
  // clamped to +-2^26 once.  Rows and keys per head stay below 2^24 (the 32-bit buffer offsets), so
  // past the clamp every slot of every tile is visible (or, for the window term, none is hidden)
  // exactly as with the unclamped value.
  const int64_t base64 = q_wg + qoff - k_lo;
  int rbase = (int)max((int64_t)-(1 << 26), min((int64_t)(1 << 26), base64));
  const int wbase = WINDOW ? (int)max((int64_t)-(1 << 26), min((int64_t)(1 << 26), base64 - window)) : 0;
  const int row_bytes = (int)(2 * ss);
  const int span = max(0, (Nk - 1) * row_bytes + T::ROW_BYTES);  // the host keeps this below 2^31
  const __amdgpu_buffer_rsrc_t kbuf =
      __builtin_amdgcn_make_buffer_rsrc((void*)((const uint16_t*)p.k + khead), 0, span, kBufferFlags);
  const __amdgpu_buffer_rsrc_t vbuf =
      __builtin_amdgcn_make_buffer_rsrc((void*)((const uint16_t*)p.v + khead), 0, span, kBufferFlags);
  int voff[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int slot = (i * NW + wave) * 64 + lane;
    const int row = slot / T::CHUNKS, pc = slot % T::CHUNKS;
    voff[i] = row * row_bytes + ((pc ^ T::swz(row)) << 4);
  }
  auto issue_tile = [&](int j, uint8_t* kdst, uint8_t* vdst) __attribute__((always_inline)) {
    issue_kv_tile<LOADS, NW>(kbuf, vbuf, voff, voff, (k_lo + tile_of(j) * BN) * row_bytes, wave, kdst, vdst);
  };
  if (n_kt > 0) issue_tile(0, ks0, vs0);

  // Q and dO fragments (B operands of S^T = K Q^T and dP^T = V dO^T): row q0 + 16*qg + li, d 32c+8g..+7.
  // D_i = sum_d dO_id O_id from the same fragment pattern of O, summed over the 4 lane groups.
  const uint16_t* qp = (const uint16_t*)p.q + qhead;
  const uint16_t* dop = (const uint16_t*)p.dout + qhead;
  const uint16_t* op = (const uint16_t*)p.o + qhead;
  vec8 qf[QG][T::DC], df[QG][T::DC];
  float lse2[QG], dlt[QG];
  auto load_qdo = [&](int q0u) __attribute__((always_inline)) {
#pragma unroll
    for (int qg = 0; qg < QG; ++qg) {
      const int qrow = min(q0u + 16 * qg + li, Nq - 1);
#pragma unroll
      for (int c = 0; c < T::DC; ++c) {
        const int64_t e = qrow * ss + 32 * c + 8 * g;
        qf[qg][c] = *(const vec8*)(qp + e);
        df[qg][c] = *(const vec8*)(dop + e);
      }
    }
  };
  auto row_values = [&](int q0u) __attribute__((always_inline)) {
#pragma unroll
    for (int qg = 0; qg < QG; ++qg) {
      const int qi = q0u + 16 * qg + li;
      const int qrow = min(qi, Nq - 1);
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < T::DC; ++c) {
        const vec8 of = *(const vec8*)(op + qrow * ss + 32 * c + 8 * g);
#pragma unroll
        for (int x = 0; x < 8; ++x) acc = __builtin_fmaf(to_f32<IS_BF16>(df[qg][c], x), to_f32<IS_BF16>(of, x), acc);
      }
      dlt[qg] = wave_sum_xor16_32(acc);
      lse2[qg] = p.lse[gm.row0 + qrow] * kLog2e;
      if (g == 0 && qi < Nq) p.delta[gm.row0 + qi] = dlt[qg];
    }
  };
  load_qdo(q0);
  row_values(q0);

  const float cexp = p.c;  // scale * log2(e), signed
  f32x4_t dqa[QG][T::DT];
#pragma unroll
  for (int qg = 0; qg < QG; ++qg)
#pragma unroll
    for (int dt = 0; dt < T::DT; ++dt) dqa[qg][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  int rb[T::DC], tb[T::DT];
  lane_offsets<D>(li, g, rb, tb);

  // sw_c: the heavy tile's last step of a pair, which loads the light tile's Q and dO fragments once its
  // own S^T and dP^T products no longer need them
  // stores_in_flight: the first step after a pair's switch, whose wait leaves the heavy tile's dQ stores
  // (issued after this tile's DMA; the memory counter retires in order) in flight
  constexpr int kDqStores = QG * T::DT / 2;
  bool stores_in_flight = false;
  auto step = [&](int j, const uint8_t* ks, const uint8_t* vs, uint8_t* kn, uint8_t* vn, auto last_c, auto sw_c)
      __attribute__((always_inline)) {
    if (stores_in_flight) {
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(kDqStores));
      stores_in_flight = false;
    } else {
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    }
    lds_barrier();
    if constexpr (!decltype(last_c)::value) issue_tile(j + 1, kn, vn);
    constexpr bool switch_unit = decltype(sw_c)::value;
    const int jt = tile_of(j);
    const int key0 = k_lo + jt * BN;
    const int dpos = rbase + wave * QW - jt * BN;  // the wave's first query position minus key0
    const int dwin = wbase + wave * QW - jt * BN;  // the same minus the window
    // the wave's 32 queries see some key of this tile; element masks where the causal edge, the window
    // edge or the chunk's end cross it
    const bool active = (!CAUSAL || dpos + QW - 1 >= 0) && (!WINDOW || dwin <= BN - 1);
    if (active) {
      const bool need_mask = (CAUSAL && dpos < BN - 1) || (key0 + BN > kv1) || (WINDOW && dwin + QW - 1 > 0);
      uint32_t dsf[QG][KC][4];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        f32x4_t s[QG], dp[QG];
#pragma unroll
        for (int qg = 0; qg < QG; ++qg) {
          s[qg] = f32x4_t{0.f, 0.f, 0.f, 0.f};
          dp[qg] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int c = 0; c < T::DC; ++c) {
          const vec8 kf = row_frag<vec8>(ks, rb[c], 16 * kt * T::ROW_BYTES);
          const vec8 vf = row_frag<vec8>(vs, rb[c], 16 * kt * T::ROW_BYTES);
#pragma unroll
          for (int qg = 0; qg < QG; ++qg) {
            s[qg] = E::mfma(kf, qf[qg][c], s[qg]);
            dp[qg] = E::mfma(vf, df[qg][c], dp[qg]);
          }
        }
        // lane holds keys key0 + 16*kt + 4*g + r for query q0 + 16*qg + li
        float a[QG][4];
#pragma unroll
        for (int qg = 0; qg < QG; ++qg)
#pragma unroll
          for (int r = 0; r < 4; ++r) a[qg][r] = __builtin_fmaf(s[qg][r], cexp, -lse2[qg]);
        if (need_mask) {
          keep_branch();
          // clamped again: slots span fewer than 128 keys, so values past +-512 hide the same slots
          const int dq0 = CAUSAL ? max(-512, min(512, dpos)) : 0;
          const int dw0 = WINDOW ? max(-512, min(512, dwin)) : 0;
          const int kend = kv1 - key0;  // slots from kend on lie past the chunk
#pragma unroll
          for (int qg = 0; qg < QG; ++qg) {
            // visible slots of this query: [lo, hi] (tiles start at the chunk's first visible key, so
            // only a window needs the lower edge; past the chunk the window is empty anyway)
            const int hi = (CAUSAL ? min(kend - 1, dq0 + 16 * qg + li) : kend - 1) - 4 * g;
            const int lo = WINDOW ? dw0 + 16 * qg + li - 4 * g : 0;
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (16 * kt + r > hi || (WINDOW && 16 * kt + r < lo)) a[qg][r] = kNegInf;
          }
        }
#pragma unroll
        for (int qg = 0; qg < QG; ++qg) {
          float ds[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) ds[r] = __builtin_amdgcn_exp2f(a[qg][r]) * (dp[qg][r] - dlt[qg]);
          const int kc = kt >> 1, half = kt & 1;
          dsf[qg][kc][2 * half + 0] = E::pack2(ds[0], ds[1]);
          dsf[qg][kc][2 * half + 1] = E::pack2(ds[2], ds[3]);
        }
      }
      if constexpr (switch_unit) load_qdo(qt_b * BM + wave * QW);
      // dQ^T += K^T dS^T
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)
#pragma unroll
        for (int dt = 0; dt < T::DT; ++dt) {
          const vec8 kt_frag = tr_frag<T::ROW_BYTES, vec8>(ks, tb[dt], 32 * kc * T::ROW_BYTES);
#pragma unroll
          for (int qg = 0; qg < QG; ++qg) dqa[qg][dt] = E::mfma(kt_frag, as_vec8<vec8>(dsf[qg][kc]), dqa[qg][dt]);
        }
    } else if constexpr (switch_unit) {
      load_qdo(qt_b * BM + wave * QW);
    }
  };

  // dQ = scale * accumulated (dS K) over the chunk's keys (0 when it sees none); lane holds d =
  // 16*dt + 4*g + r of query q0s + 16*qg + li.  16-byte stores: lanes 16 apart (the same row) exchange the
  // pieces of two d tiles, so each store writes 64 contiguous bytes of 16 rows (as the forward's output)
  uint16_t* dqp = (uint16_t*)p.dq + qhead;
  auto store_dq = [&](int q0s) __attribute__((always_inline)) {
    const bool odd = (g & 1) != 0;
#pragma unroll
    for (int qg = 0; qg < QG; ++qg) {
      const int qi = q0s + 16 * qg + li;
#pragma unroll
      for (int m = 0; m < T::DT / 2; ++m) {
        const f32x4_t x0 = dqa[qg][2 * m] * p.scale, x1 = dqa[qg][2 * m + 1] * p.scale;
        const uint32_t a0 = E::pack2(x0[0], x0[1]), a1 = E::pack2(x0[2], x0[3]);
        const uint32_t b0 = E::pack2(x1[0], x1[1]), b1 = E::pack2(x1[2], x1[3]);
        const uint32_t s0 = odd ? a0 : b0, s1 = odd ? a1 : b1;
        const uint32_t r0 = __shfl_xor(s0, 16), r1 = __shfl_xor(s1, 16);
        const u32x4_t w = odd ? u32x4_t{r0, r1, b0, b1} : u32x4_t{a0, a1, r0, r1};
        const int col = odd ? 16 * (2 * m + 1) + 4 * (g - 1) : 16 * (2 * m) + 4 * g;
        // (pairs: every row is real, and every store must issue: the next step's wait counts them)
        if (PAIR || qi < Nq) *(u32x4_t*)(dqp + qi * ss + col) = w;
      }
    }
  };

  const std::integral_constant<bool, false> more, stay;
  const std::integral_constant<bool, true> last, switch_c;
  if constexpr (PAIR) {
    // both tiles stream an even number of key tiles (128-query tiles of 64-key tiles, a key count that is
    // a multiple of 128), so the light tile starts in stage 0; the heavy tile's last step prefetches its
    // first K/V tile
    int j = 0;
    for (; j + 2 < n_kt_a; j += 2) {
      step(j, ks0, vs0, ks1, vs1, more, stay);
      step(j + 1, ks1, vs1, ks0, vs0, more, stay);
    }
    step(j, ks0, vs0, ks1, vs1, more, stay);
    step(j + 1, ks1, vs1, ks0, vs0, more, switch_c);
    j += 2;
    // the light tile's row values first (their loads are waited for at once), then the heavy tile's dQ,
    // whose stores the light tile's first step leaves in flight
    const int q0_heavy = q0;
    q_wg = qt_b * BM;
    q0 = q_wg + wave * QW;
    rbase = q_wg;  // the whole problem: no offset, keys from 0
    row_values(q0);
    store_dq(q0_heavy);
#pragma unroll
    for (int qg = 0; qg < QG; ++qg)
#pragma unroll
      for (int dt = 0; dt < T::DT; ++dt) dqa[qg][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    stores_in_flight = true;  // (cleared by the light tile's first step)
    for (; j + 2 < n_kt; j += 2) {
      step(j, ks0, vs0, ks1, vs1, more, stay);
      step(j + 1, ks1, vs1, ks0, vs0, more, stay);
    }
    step(j, ks0, vs0, ks1, vs1, more, stay);
    step(j + 1, ks1, vs1, ks0, vs0, last, stay);
  } else if (n_kt > 0) {
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
  store_dq(q0);
}

// ------------------------------------------------------------------------------------------------
// dK, dV : one workgroup per (b, h, 128-key tile)
// ------------------------------------------------------------------------------------------------
// ATOMIC_DQ (the atomic mode, fa_bwd_atomic): the workgroup also forms dQ's part of its 128 keys from the
// dS it computes, dQ_i += sum_j dS_ij k_j, and adds it into the fp32 accumulator p.dq_acc with global atomics
// (the per-step sums of different workgroups arrive in any order, so the result can differ in the last
// bits from run to run).  Per 32-query step every wave writes its dS (rounded as for dK) transposed into
// LDS, and after a barrier each wave multiplies the whole step's dS by K (staged once in LDS) for its
// share of dQ's 16 x 16 tiles.
// PAIR (whole causal problems with an even number of 128-key tiles, deterministic mode): workgroup r runs
// the heavy key tile r and then the light key tile n-1-r of one head over one continuous Q/dO stream, so
// every workgroup has the same work; the heavy tile's last step prefetches the light tile's first Q/dO
// tile and loads its K and V once its own S and dP products are done.
template <int D, bool IS_BF16, bool CAUSAL, bool WINDOW, bool VARLEN, int NW, int KW, int MINB, bool ATOMIC_DQ = false,
          bool PAIR = false>
__global__ __launch_bounds__(NW * 64, MINB) void fa_bwd_dkdv(BwdParams p) {
  typedef BwdTile<D> T;
  typedef Elem<IS_BF16> E;
  typedef typename E::vec8 vec8;
  constexpr int BK = NW * KW;                       // keys per workgroup (NW waves of KW keys)
  static_assert(BK == 128, "the launch grid has one workgroup per 128 keys");
  constexpr int BQ = 64, QS = 32;                   // queries per LDS tile, per step
  constexpr int KG = KW / 16, QGS = QS / 16;
  constexpr int TILE_BYTES = BQ * T::ROW_BYTES;
  constexpr int LOADS = TILE_BYTES / (16 * 64 * NW);
  __shared__ __attribute__((aligned(1024))) uint8_t qs0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t qs1[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t os0[TILE_BYTES];  // dO
  __shared__ __attribute__((aligned(1024))) uint8_t os1[TILE_BYTES];
  // per-row values of a Q tile: lse * log2(e) in [0, BQ), D in [BQ, 2 BQ); +inf / 0 past the end
  __shared__ __attribute__((aligned(16))) float rv0[2 * BQ];
  __shared__ __attribute__((aligned(16))) float rv1[2 * BQ];
  static_assert(BQ == 64, "one lane of one wave loads each row value");
  // atomic mode: the workgroup's K rows (swizzled as the Q/dO tiles) and two buffers of one step's dS^T
  // (128 keys x 32 queries, one 64-byte row per key)
  constexpr int KS_BYTES = ATOMIC_DQ ? BK * T::ROW_BYTES : 16;
  constexpr int DS_ROW = QS * 2, DS_BYTES = ATOMIC_DQ ? BK * DS_ROW : 16;
  __shared__ __attribute__((aligned(1024))) uint8_t ks_l[KS_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t dst0[DS_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t dst1[DS_BYTES];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, li = lane & 15;
  static_assert(!PAIR || (CAUSAL && !WINDOW && !VARLEN && !ATOMIC_DQ), "pairs are for whole causal problems");
  int bh, kt, kt_b = -1;
  if constexpr (VARLEN) {
    unit_of_spread(blockIdx.x, p.n_tiles_k, false, bh, kt);
    if (bh >= p.B * p.H) return;  // padding head of the grid
  } else if constexpr (PAIR) {
    int r;  // pair r of a head: key tiles r and n-1-r (n_tiles_k counts pairs)
    unit_of(blockIdx.x, p.n_units_k, p.n_tiles_k, false, bh, r);
    kt = r;
    kt_b = 2 * p.n_tiles_k - 1 - r;
  } else {
    unit_of(blockIdx.x, p.n_units_k, p.n_tiles_k, false, bh, kt);  // causal: the chunk's first key tile first
  }
  const int b = bh / p.H, h = bh - (bh / p.H) * p.H;
  const BwdGeom gm = bwd_geometry<VARLEN, CAUSAL>(p, b, h, bh);
  if (VARLEN && (gm.skip || kt * BK >= gm.Nk)) return;  // a bad sequence, or a tile past its end
  const int Nq = gm.Nq;
  const int64_t qoff = gm.qoff, window = gm.window;
  const int kv1 = gm.kv1;  // keys of the chunk: [gm.kv0, kv1)
  int k_wg = gm.kv0 + kt * BK, kw0 = k_wg + wave * KW;  // (the light tile's, after a pair's switch)
  const int64_t qhead = gm.qhead, khead = gm.khead;
  const int64_t ss = p.stride_s;

  // K and V of the wave's keys as B operands of S = Q K^T and dP = dO V^T: lane holds key kw0 + 16*kg + li,
  // d 32c + 8g .. +7; keys past the chunk are zero (their gradients are not stored)
  const uint16_t* kp = (const uint16_t*)p.k + khead;
  const uint16_t* vp = (const uint16_t*)p.v + khead;
  vec8 kf[KG][T::DC], vf[KG][T::DC];
  auto load_kv = [&](int kw0u) __attribute__((always_inline)) {
#pragma unroll
    for (int kg = 0; kg < KG; ++kg) {
      const int key = kw0u + 16 * kg + li;
      const int krow = min(key, kv1 - 1);
#pragma unroll
      for (int c = 0; c < T::DC; ++c) {
        const int64_t e = krow * ss + 32 * c + 8 * g;
        u32x4_t kr = *(const u32x4_t*)(kp + e), vr = *(const u32x4_t*)(vp + e);
        if (key >= kv1) kr = vr = u32x4_t{0u, 0u, 0u, 0u};
        kf[kg][c] = __builtin_bit_cast(vec8, kr);
        vf[kg][c] = __builtin_bit_cast(vec8, vr);
      }
    }
  };
  load_kv(kw0);
  if constexpr (ATOMIC_DQ) {  // published to the other waves by the first step's barrier
#pragma unroll
    for (int kg = 0; kg < KG; ++kg) {
      const int row = wave * KW + 16 * kg + li;
#pragma unroll
      for (int c = 0; c < T::DC; ++c)
        *(vec8*)(ks_l + row * T::ROW_BYTES + (((4 * c + g) ^ T::swz(row)) << 4)) = kf[kg][c];
    }
  }

  // Q/dO tiles of BQ rows from i_begin: the query rows that see some key of this workgroup (causal: from
  // the first key's position; window: up to the last key's position plus the window)
  const int i_begin = CAUSAL ? (int)min((int64_t)Nq, max((int64_t)0, k_wg - qoff)) : 0;
  const int i_last = WINDOW ? (int)min((int64_t)Nq - 1, k_wg + BK - 1 + window - qoff) : Nq - 1;
  const int n_qt_a = i_last >= i_begin ? (i_last - i_begin) / BQ + 1 : 0;
  // a pair's light key tile: the query rows from its first key on (the whole problem: no offset)
  const int i_begin_b = PAIR ? min(Nq, kt_b * BK) : 0;
  const int n_qt_b = PAIR ? (Nq - 1 - i_begin_b) / BQ + 1 : 0;
  const int n_qt = n_qt_a + n_qt_b;
  // first query row of tile j of the stream: the first key tile's tiles, then the light tile's
  auto row_of = [&](int j) __attribute__((always_inline)) {
    return PAIR && j >= n_qt_a ? i_begin_b + (j - n_qt_a) * BQ : i_begin + j * BQ;
  };
  // positions in 32 bits: row 0's position minus k_wg, clamped to +-2^26 once, and the window
  // corrected by what the clamp removed, clamped to +-2^27.  Rows per head stay below 2^24 (the
  // 32-bit buffer offsets): past +2^26 every row sees every key causally, below -2^26 no row is
  // processed, and the corrected window compares with the clamped positions as the window with the
  // exact ones.
  const int64_t rb64 = qoff - k_wg;
  const int64_t rbc64 = max((int64_t)-(1 << 26), min((int64_t)(1 << 26), rb64));
  int rbase = (int)rbc64;
  const int wv = WINDOW ? (int)max((int64_t)-(1 << 27), min((int64_t)(1 << 27), window - (rb64 - rbc64))) : 0;
  const int row_bytes = (int)(2 * ss);
  const int span = max(0, (Nq - 1) * row_bytes + T::ROW_BYTES);
  const __amdgpu_buffer_rsrc_t qbuf =
      __builtin_amdgcn_make_buffer_rsrc((void*)((const uint16_t*)p.q + qhead), 0, span, kBufferFlags);
  const __amdgpu_buffer_rsrc_t obuf =
      __builtin_amdgcn_make_buffer_rsrc((void*)((const uint16_t*)p.dout + qhead), 0, span, kBufferFlags);
  int voff[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int slot = (i * NW + wave) * 64 + lane;
    const int row = slot / T::CHUNKS, pc = slot % T::CHUNKS;
    voff[i] = row * row_bytes + ((pc ^ T::swz(row)) << 4);
  }
  auto issue_tile = [&](int j, uint8_t* qdst, uint8_t* odst) __attribute__((always_inline)) {
    issue_kv_tile<LOADS, NW>(qbuf, obuf, voff, voff, row_of(j) * row_bytes, wave, qdst, odst);
  };
  if (n_qt > 0) issue_tile(0, qs0, os0);

  const float cexp = p.c;
  const float* lse_h = p.lse + gm.row0;
  const float* dlt_h = p.delta + gm.row0;
  // row values of tile jt for this lane's row (wave 0 only)
  auto load_rows = [&](int jt, float& l2v, float& dv) __attribute__((always_inline)) {
    const int qi = row_of(jt) + lane;
    if (qi < Nq) {
      l2v = lse_h[qi] * kLog2e;
      dv = dlt_h[qi];
    } else {
      l2v = kPosInf;
      dv = 0.f;
    }
  };
  if (wave == 0 && n_qt > 0) {
    float a, d;
    load_rows(0, a, d);
    rv0[lane] = a;
    rv0[BQ + lane] = d;
  }
  f32x4_t dka[KG][T::DT], dva[KG][T::DT];
#pragma unroll
  for (int kg = 0; kg < KG; ++kg)
#pragma unroll
    for (int dt = 0; dt < T::DT; ++dt) {
      dka[kg][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      dva[kg][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
  int rb[T::DC], tb[T::DT];
  lane_offsets<D>(li, g, rb, tb);

  // atomic mode, one 32-query step: publish this wave's dS^T rows, then form this wave's dQ tiles over the
  // workgroup's 128 keys, dQ[q][d] = sum_k dS[q][k] K[k][d] (A = dS from dS^T by transposing reads, B =
  // K^T from the K rows by transposing reads, both with the key order of tr_frag), and add them to dq_acc.
  // Tiles (16 queries x 16 d): QGS * DT of them, NW waves; wave w takes query group w / (NW / QGS) and d
  // tiles of its share.  The dS buffers alternate between steps, so one barrier per step suffices: a
  // buffer is rewritten only after the next step's barrier, which follows every wave's reads of it.
  float* dq_acc = p.dq_acc;
  constexpr int WPQ = NW / QGS;     // waves per query group of a step
  constexpr int DTW = T::DT / WPQ;  // dQ d tiles per wave (2 for D = 128, 1 for D = 64)
  static_assert(DTW >= 1 && DTW * WPQ == T::DT, "dQ tiles split evenly over the waves");
  // the wave's query group and first d tile; K^T read offsets computed here, not indexed from tb[] by a
  // wave-dependent index (which would place tb[] in private memory)
  // The offsets are made opaque to the optimizer: split into a chain of address steps, an LDS read can end
  // up too many steps from its LDS object for the compiler to prove it apart from the Q/dO tile DMA, which
  // then costs a wait for that DMA before the read.
  const int dq_qg = wave / WPQ, dq_dt0 = (wave % WPQ) * DTW;
  int ktb[DTW];
#pragma unroll
  for (int t = 0; t < DTW; ++t) {
    ktb[t] = tr_offset<D>(li, g, dq_dt0 + t);
    asm("" : "+v"(ktb[t]));
  }
  // dS^T lane offset: row 4g + (li >> 2) (a key), column 16 qg + 4 (li & 3) (queries)
  int ds_off = (4 * g + (li >> 2)) * DS_ROW + (16 * dq_qg + 4 * (li & 3)) * 2;
  asm("" : "+v"(ds_off));
  auto atomic_dq_step = [&](uint8_t* dst, const uint32_t (&dsq)[KG][4], int qh0) __attribute__((always_inline)) {
    if constexpr (ATOMIC_DQ) {
#pragma unroll
      for (int kg = 0; kg < KG; ++kg) {  // key row wave*KW + 16 kg + li: queries 4g..4g+3 and 16+4g..16+4g+3
        uint8_t* row = dst + (wave * KW + 16 * kg + li) * DS_ROW;
        *(u32x2_t*)(row + 8 * g) = u32x2_t{dsq[kg][0], dsq[kg][1]};
        *(u32x2_t*)(row + 32 + 8 * g) = u32x2_t{dsq[kg][2], dsq[kg][3]};
      }
      lds_barrier();
      f32x4_t acc[DTW];
#pragma unroll
      for (int t = 0; t < DTW; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < BK / 32; ++kc) {
        const vec8 a = tr_frag<DS_ROW, vec8>(dst, ds_off, 32 * kc * DS_ROW);
#pragma unroll
        for (int t = 0; t < DTW; ++t) {
          const vec8 bk = tr_frag<T::ROW_BYTES, vec8>(ks_l, ktb[t], 32 * kc * T::ROW_BYTES);
          acc[t] = E::mfma(a, bk, acc[t]);
        }
      }
      // lane holds dQ rows qh0 + 16 qg + 4 g + r, column 16 (dt0 + t) + li.  Every lane issues every atomic
      // (a row past the end adds 0 to the last row), so a step always issues 4 DTW of them
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int qi = qh0 + 16 * dq_qg + 4 * g + r;
        float* dst_row = dq_acc + qhead + min(qi, Nq - 1) * ss;
#pragma unroll
        for (int t = 0; t < DTW; ++t) unsafeAtomicAdd(dst_row + 16 * (dq_dt0 + t) + li, qi < Nq ? acc[t][r] : 0.f);
      }
    }
  };
  // atomic instructions a wave issues per Q/dO tile (both 32-query steps)
  constexpr int kAtomicsPerTile = ATOMIC_DQ ? (BQ / QS) * 4 * DTW : 0;
  // store instructions of store_dkdv (dK and dV, 16 bytes per lane)
  constexpr int kDkdvStores = KG * T::DT;
  bool stores_in_flight = false;

  // sw_c: the heavy key tile's last step of a pair, which loads the light tile's K and V once its last
  // S and dP products no longer need them
  auto step = [&](int j, const uint8_t* qs, const uint8_t* os, const float* rv, uint8_t* qn, uint8_t* on, float* rvn,
                  auto last_c, auto sw_c) __attribute__((always_inline)) {
    constexpr bool switch_unit = decltype(sw_c)::value;
    // this wave's share of tile j has landed (the atomic mode leaves the previous tile's atomics, issued after
    // tile j's DMA, in flight; the first step after a pair's switch leaves the heavy tile's dK/dV stores, issued
    // after them, in flight too: the memory counter retires in order)
    if (stores_in_flight) {
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(kAtomicsPerTile + kDkdvStores));
      stores_in_flight = false;
    } else if (ATOMIC_DQ && j > 0) {
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(kAtomicsPerTile));
    } else {
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    }
    lds_barrier();
    // the next tile's row values are loaded before its DMA is issued (the memory counter retires in
    // order) and stored to LDS after this tile's work, for the next barrier to publish
    float nl = 0.f, nd = 0.f;
    if constexpr (!decltype(last_c)::value) {
      if (wave == 0) load_rows(j + 1, nl, nd);
      issue_tile(j + 1, qn, on);
    }
    const int tile0 = row_of(j);
#pragma unroll
    for (int hh = 0; hh < BQ / QS; ++hh) {
      const int qh0 = tile0 + QS * hh;  // first query row of this step
      const int c = qh0 + rbase - wave * KW;  // its position minus the wave's first key
      // some query of the step sees some key of the wave (causal: the last query is not before the
      // first key; window: the first query is not past the last key's window)
      const bool active = qh0 < Nq && (!CAUSAL || c + QS - 1 >= 0) && (!WINDOW || c <= KW - 1 + wv);
      uint32_t dsq[KG][4];  // atomic mode: this wave's dS of the step (0 when the wave skips it)
      if constexpr (ATOMIC_DQ) {
#pragma unroll
        for (int kg = 0; kg < KG; ++kg)
#pragma unroll
          for (int i = 0; i < 4; ++i) dsq[kg][i] = 0u;
      }
      if (active) {
        const bool need_mask = (CAUSAL && c < KW - 1) || (WINDOW && c + QS - 1 > wv);
        // the wave's first key minus the step's first row position (plus the window), clamped: lanes
        // span fewer than 64 keys and rows, so values past +-512 hide the same rows
        const int dk0 = CAUSAL ? max(-512, min(512, -c)) : 0;
        const int dkw = WINDOW ? max(-512, min(512, wv - c)) : 0;
        // LDS fragments are read ahead of their products: the Q and dO rows of (qq, c) pair f + RA while
        // pair f's products run; the transposed dO and Q of d-tiles 0..TA-1 before the last query group's
        // exponentials, then those of d-tile dt + TA while dt's products run.  A scheduling barrier after
        // each group of reads keeps the compiler from moving them back down to their uses.
        constexpr int NR = QGS * T::DC, RA = 3, TA = 3;
        const int hrow = QS * hh * T::ROW_BYTES;
        vec8 rq[RA], ro[RA], tq[TA], to[TA];
        auto read_rows = [&](int f, vec8& a, vec8& b) __attribute__((always_inline)) {
          const int off = hrow + 16 * (f / T::DC) * T::ROW_BYTES;
          a = row_frag<vec8>(qs, rb[f % T::DC], off);
          b = row_frag<vec8>(os, rb[f % T::DC], off);
        };
        auto read_tr = [&](int dt, vec8& a, vec8& b) __attribute__((always_inline)) {
          a = tr_frag<T::ROW_BYTES, vec8>(os, tb[dt], hrow);
          b = tr_frag<T::ROW_BYTES, vec8>(qs, tb[dt], hrow);
        };
#pragma unroll
        for (int f = 0; f < RA; ++f) read_rows(f, rq[f], ro[f]);
        uint32_t pp[KG][4], dsp[KG][4];
#pragma unroll
        for (int qq = 0; qq < QGS; ++qq) {
          f32x4_t s[KG], dp[KG];
#pragma unroll
          for (int kg = 0; kg < KG; ++kg) {
            s[kg] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            dp[kg] = f32x4_t{0.f, 0.f, 0.f, 0.f};
          }
#pragma unroll
          for (int c = 0; c < T::DC; ++c) {
            const int f = qq * T::DC + c;
            const vec8 qa = rq[f % RA], oa = ro[f % RA];
            if (f + RA < NR) read_rows(f + RA, rq[f % RA], ro[f % RA]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int kg = 0; kg < KG; ++kg) {
              s[kg] = E::mfma(qa, kf[kg][c], s[kg]);
              dp[kg] = E::mfma(oa, vf[kg][c], dp[kg]);
            }
          }
          // lane holds queries qh0 + 16*qq + 4*g + r for key kw0 + 16*kg + li
          const f32x4_t l2 = *(const f32x4_t*)(rv + QS * hh + 16 * qq + 4 * g);
          const f32x4_t dl = *(const f32x4_t*)(rv + BQ + QS * hh + 16 * qq + 4 * g);
          if (qq == QGS - 1) {  // after the row values, which the exponentials wait for
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int dt = 0; dt < TA; ++dt) read_tr(dt, to[dt], tq[dt]);
            __builtin_amdgcn_sched_barrier(0);
          }
          float a[KG][4];
#pragma unroll
          for (int kg = 0; kg < KG; ++kg)
#pragma unroll
            for (int r = 0; r < 4; ++r) a[kg][r] = __builtin_fmaf(s[kg][r], cexp, -l2[r]);
          if (need_mask) {
            keep_branch();
#pragma unroll
            for (int kg = 0; kg < KG; ++kg) {
              // the lane's key minus its first row's position is rel = dk0 + 16 kg + li - 16 qq - 4 g;
              // hidden rows r: before the key (r < rel, causal) or more than `window` after it
              const int rl = 16 * kg + li - 16 * qq - 4 * g;
              const int lo = CAUSAL ? max(-1, min(4, dk0 + rl)) : -1;  // rows r < lo
              const int hi = WINDOW ? max(-1, min(4, dkw + rl)) : 4;   // rows r > hi
#pragma unroll
              for (int r = 0; r < 4; ++r)
                if (r < lo || r > hi) a[kg][r] = kNegInf;
            }
          }
#pragma unroll
          for (int kg = 0; kg < KG; ++kg) {
            float pr[4], ds[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              pr[r] = __builtin_amdgcn_exp2f(a[kg][r]);
              ds[r] = pr[r] * (dp[kg][r] - dl[r]);
            }
            pp[kg][2 * qq + 0] = E::pack2(pr[0], pr[1]);
            pp[kg][2 * qq + 1] = E::pack2(pr[2], pr[3]);
            dsp[kg][2 * qq + 0] = E::pack2(ds[0], ds[1]);
            dsp[kg][2 * qq + 1] = E::pack2(ds[2], ds[3]);
          }
        }
        if constexpr (switch_unit) {
          if (hh == BQ / QS - 1) load_kv(kt_b * BK + wave * KW);
        }
        // dV^T += dO^T P ;  dK^T += Q^T dS  (k index over this step's 32 queries)
#pragma unroll
        for (int dt = 0; dt < T::DT; ++dt) {
          const vec8 ot = to[dt % TA], qtf = tq[dt % TA];
          if (dt + TA < T::DT) read_tr(dt + TA, to[dt % TA], tq[dt % TA]);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int kg = 0; kg < KG; ++kg) {
            dva[kg][dt] = E::mfma(ot, as_vec8<vec8>(pp[kg]), dva[kg][dt]);
            dka[kg][dt] = E::mfma(qtf, as_vec8<vec8>(dsp[kg]), dka[kg][dt]);
          }
        }
        if constexpr (ATOMIC_DQ) {
#pragma unroll
          for (int kg = 0; kg < KG; ++kg)
#pragma unroll
            for (int i = 0; i < 4; ++i) dsq[kg][i] = dsp[kg][i];
        }
      } else if constexpr (switch_unit) {
        if (hh == BQ / QS - 1) load_kv(kt_b * BK + wave * KW);
      }
      if constexpr (ATOMIC_DQ) atomic_dq_step(hh & 1 ? dst1 : dst0, dsq, qh0);
    }
    if constexpr (!decltype(last_c)::value) {
      if (wave == 0) {
        rvn[lane] = nl;
        rvn[BQ + lane] = nd;
      }
    }
  };

  // dK = scale * accumulated (dS^T Q), dV (0 for keys no query sees): lane holds d = 16*dt + 4*g + r of
  // key kw0 + 16*kg + li; rows outside the chunk are left as they are
  uint16_t* dkp = (uint16_t*)p.dk + khead;
  uint16_t* dvp = (uint16_t*)p.dv + khead;
  // (16-byte stores: lanes 16 apart, the same key, exchange the pieces of two d tiles, as in the forward)
  auto store_dkdv = [&]() __attribute__((always_inline)) {
    const bool odd = (g & 1) != 0;
    auto put = [&](uint16_t* base, int key, f32x4_t x0, f32x4_t x1, int m) __attribute__((always_inline)) {
      const uint32_t a0 = E::pack2(x0[0], x0[1]), a1 = E::pack2(x0[2], x0[3]);
      const uint32_t b0 = E::pack2(x1[0], x1[1]), b1 = E::pack2(x1[2], x1[3]);
      const uint32_t s0 = odd ? a0 : b0, s1 = odd ? a1 : b1;
      const uint32_t r0 = __shfl_xor(s0, 16), r1 = __shfl_xor(s1, 16);
      const u32x4_t w = odd ? u32x4_t{r0, r1, b0, b1} : u32x4_t{a0, a1, r0, r1};
      const int col = odd ? 16 * (2 * m + 1) + 4 * (g - 1) : 16 * (2 * m) + 4 * g;
      // (pairs: every key is real, and every store must issue: the next step's wait counts them)
      if (PAIR || key < kv1) *(u32x4_t*)(base + key * ss + col) = w;
    };
#pragma unroll
    for (int kg = 0; kg < KG; ++kg) {
      const int key = kw0 + 16 * kg + li;
#pragma unroll
      for (int m = 0; m < T::DT / 2; ++m) {
        put(dkp, key, dka[kg][2 * m] * p.scale, dka[kg][2 * m + 1] * p.scale, m);
        put(dvp, key, dva[kg][2 * m], dva[kg][2 * m + 1], m);
      }
    }
  };

  const std::integral_constant<bool, false> more, stay;
  const std::integral_constant<bool, true> last, switch_c;
  if constexpr (PAIR) {
    // both key tiles stream an even number of 64-row Q/dO tiles (a query count that is a multiple of
    // 128), so the light tile starts in stage 0; the heavy tile's last step prefetches its first one
    int j = 0;
    for (; j + 2 < n_qt_a; j += 2) {
      step(j, qs0, os0, rv0, qs1, os1, rv1, more, stay);
      step(j + 1, qs1, os1, rv1, qs0, os0, rv0, more, stay);
    }
    step(j, qs0, os0, rv0, qs1, os1, rv1, more, stay);
    step(j + 1, qs1, os1, rv1, qs0, os0, rv0, more, switch_c);
    j += 2;
    store_dkdv();
    stores_in_flight = true;  // (cleared by the light tile's first step)
    k_wg = kt_b * BK;
    kw0 = k_wg + wave * KW;
    rbase = -k_wg;  // row 0's position minus the light tile's first key (no offset)
#pragma unroll
    for (int kg = 0; kg < KG; ++kg)
#pragma unroll
      for (int dt = 0; dt < T::DT; ++dt) {
        dka[kg][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        dva[kg][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
    for (; j + 2 < n_qt; j += 2) {
      step(j, qs0, os0, rv0, qs1, os1, rv1, more, stay);
      step(j + 1, qs1, os1, rv1, qs0, os0, rv0, more, stay);
    }
    step(j, qs0, os0, rv0, qs1, os1, rv1, more, stay);
    step(j + 1, qs1, os1, rv1, qs0, os0, rv0, last, stay);
  } else if (n_qt > 0) {
    int j = 0;
    for (; j + 2 < n_qt; j += 2) {
      step(j, qs0, os0, rv0, qs1, os1, rv1, more, stay);
      step(j + 1, qs1, os1, rv1, qs0, os0, rv0, more, stay);
    }
    if (j + 2 == n_qt) {
      step(j, qs0, os0, rv0, qs1, os1, rv1, more, stay);
      step(j + 1, qs1, os1, rv1, qs0, os0, rv0, last, stay);
    } else {
      step(j, qs0, os0, rv0, qs1, os1, rv1, last, stay);
    }
  }
  store_dkdv();
}

// ------------------------------------------------------------------------------------------------
// atomic mode: D and the zeroed accumulator before the dK/dV kernel, dq from the accumulator after it
// ------------------------------------------------------------------------------------------------
// Four lanes per query row (64 rows per 256-thread block, grid-stride): D_i = sum_d dO_id O_id and the row of dq_acc set
// to 0.  Lane g takes d = 32c + 8g .. +7 for every c and the four partial sums are combined pairwise, the
// order in which fa_bwd_dq forms D, so both modes hold the same D bit for bit.
template <int D, bool IS_BF16>
__global__ __launch_bounds__(256) void fa_bwd_prep(BwdParams p) {
  typedef typename Elem<IS_BF16>::vec8 vec8;
  const int g = threadIdx.x & 3;
  const int64_t rows = (int64_t)p.B * p.H * p.Nq;
  // the 4 lanes of a row run the same iterations
  for (int64_t row = (int64_t)blockIdx.x * 64 + (threadIdx.x >> 2); row < rows; row += (int64_t)gridDim.x * 64) {
    const int64_t bh = row / p.Nq, i = row - bh * p.Nq;
    const int64_t b = bh / p.H, h = bh - b * p.H;
    const int64_t e0 = b * p.stride_b_q + h * p.stride_h_q + i * p.stride_s + 8 * g;
    float acc = 0.f;
#pragma unroll
    for (int c = 0; c < D / 32; ++c) {
      const int64_t e = e0 + 32 * c;
      const vec8 o = *(const vec8*)((const uint16_t*)p.o + e);
      const vec8 d = *(const vec8*)((const uint16_t*)p.dout + e);
#pragma unroll
      for (int x = 0; x < 8; ++x) acc = __builtin_fmaf(to_f32<IS_BF16>(d, x), to_f32<IS_BF16>(o, x), acc);
      *(f32x4_t*)(p.dq_acc + e) = f32x4_t{0.f, 0.f, 0.f, 0.f};
      *(f32x4_t*)(p.dq_acc + e + 4) = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    acc += __shfl_xor(acc, 1, 4);
    acc += __shfl_xor(acc, 2, 4);
    if (g == 0) p.delta[row] = acc;
  }
}

// dq = scale * dq_acc, rounded to the 16-bit type; 8 elements per thread and step of a grid-stride loop
// (dq and dq_acc are dense and share a layout).
template <bool IS_BF16>
__global__ __launch_bounds__(256) void fa_bwd_dq_convert(BwdParams p, int64_t n8) {
  typedef Elem<IS_BF16> E;
  for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < n8; t += (int64_t)gridDim.x * 256) {
    const f32x4_t a = *(const f32x4_t*)(p.dq_acc + 8 * t) * p.scale;
    const f32x4_t b = *(const f32x4_t*)(p.dq_acc + 8 * t + 4) * p.scale;
    *(u32x4_t*)((uint16_t*)p.dq + 8 * t) =
        u32x4_t{E::pack2(a[0], a[1]), E::pack2(a[2], a[3]), E::pack2(b[0], b[1]), E::pack2(b[2], b[3])};
  }
}

// blocks of a grid-stride launch: enough to fill the chip many times over, at most 2^20
inline unsigned stride_grid(int64_t items, int per_block) {
  return (unsigned)std::min<int64_t>((items + per_block - 1) / per_block, (int64_t)1 << 20);
}

template <int D, bool IS_BF16, bool CAUSAL>
hipError_t launch_bwd_atomic_t(BwdParams p, hipStream_t stream) {
  const int64_t rows = (int64_t)p.B * p.H * p.Nq;
  hipLaunchKernelGGL((fa_bwd_prep<D, IS_BF16>), dim3(stride_grid(rows, 64)), dim3(256), 0, stream, p);
  p.n_tiles_k = (p.kv_len + 127) / 128;
  p.n_units_k = p.n_tiles_k * p.B * p.H;
  hipLaunchKernelGGL((fa_bwd_dkdv<D, IS_BF16, CAUSAL, false, false, kDkdvWaves, kDkdvKeys, kDkdvMinBlocks, true>),
                     dim3(p.n_units_k), dim3(64 * kDkdvWaves), 0, stream, p);
  const int64_t n8 = rows * D / 8;
  hipLaunchKernelGGL((fa_bwd_dq_convert<IS_BF16>), dim3(stride_grid(n8, 256)), dim3(256), 0, stream, p, n8);
  return hipGetLastError();
}

template <int D, bool IS_BF16, bool CAUSAL, bool WINDOW>
hipError_t launch_bwd_t(BwdParams p, hipStream_t stream) {
  p.n_tiles_q = (p.Nq + 127) / 128;
  p.n_units_q = p.B * p.H * p.n_tiles_q;
  p.n_tiles_k = (p.kv_len + 127) / 128;
  p.n_units_k = p.B * p.H * p.n_tiles_k;
  // the whole causal problem with an even number of 128-query tiles and a key count that is a multiple of
  // 128: the dQ kernel pairs its heavy and light tiles
  const bool pairs = CAUSAL && !WINDOW && p.q_offset == 0 && p.kv_start == 0 && p.kv_len == p.Nk &&
                     p.Nq == p.Nk && p.Nq % 128 == 0 && p.n_tiles_q % 2 == 0;
  if constexpr (CAUSAL && !WINDOW) {
    if (pairs) {
      BwdParams pp = p;
      pp.n_tiles_q = p.n_tiles_q / 2;
      pp.n_units_q = p.B * p.H * pp.n_tiles_q;
      hipLaunchKernelGGL((fa_bwd_dq<D, IS_BF16, true, false, false, true>), dim3(pp.n_units_q), dim3(256), 0, stream,
                         pp);
    }
  }
  if (!pairs) {
    hipLaunchKernelGGL((fa_bwd_dq<D, IS_BF16, CAUSAL, WINDOW, false>), dim3(p.n_units_q), dim3(256), 0, stream, p);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.n_units_k == 0) return e;
  // the dK/dV kernel pairs its heavy and light key tiles under the same condition (N_k = N_q)
  if constexpr (CAUSAL && !WINDOW) {
    if (pairs) {
      BwdParams pp = p;
      pp.n_tiles_k = p.n_tiles_k / 2;
      pp.n_units_k = p.B * p.H * pp.n_tiles_k;
      hipLaunchKernelGGL(
          (fa_bwd_dkdv<D, IS_BF16, true, false, false, kDkdvWaves, kDkdvKeys, kDkdvMinBlocks, false, true>),
          dim3(pp.n_units_k), dim3(64 * kDkdvWaves), 0, stream, pp);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((fa_bwd_dkdv<D, IS_BF16, CAUSAL, WINDOW, false, kDkdvWaves, kDkdvKeys, kDkdvMinBlocks>),
                     dim3(p.n_units_k), dim3(64 * kDkdvWaves), 0, stream, p);
  return hipGetLastError();
}

// packed sequences: the grid covers the longest query (key) count for every head, heads spread over the
// XCDs and padded to a multiple of 8
template <int D, bool IS_BF16, bool CAUSAL>
hipError_t launch_bwd_varlen_t(BwdParams p, hipStream_t stream) {
  const int heads = (p.B * p.H + 7) / 8 * 8;
  p.n_tiles_q = (p.Nq + 127) / 128;
  p.n_units_q = heads * p.n_tiles_q;
  p.n_tiles_k = (p.Nk + 127) / 128;
  p.n_units_k = heads * p.n_tiles_k;
  hipLaunchKernelGGL((fa_bwd_dq<D, IS_BF16, CAUSAL, false, true>), dim3(p.n_units_q), dim3(256), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((fa_bwd_dkdv<D, IS_BF16, CAUSAL, false, true, kDkdvWaves, kDkdvKeys, kDkdvMinBlocks>),
                     dim3(p.n_units_k), dim3(64 * kDkdvWaves), 0, stream, p);
  return hipGetLastError();
}

template <int D, bool IS_BF16>
hipError_t launch_bwd_c(const BwdParams& p, bool causal, hipStream_t stream) {
  if (!causal) return launch_bwd_t<D, IS_BF16, false, false>(p, stream);
  return p.window >= 0 ? launch_bwd_t<D, IS_BF16, true, true>(p, stream) : launch_bwd_t<D, IS_BF16, true, false>(p, stream);
}

}  // namespace

hipError_t launch_bwd_atomic(const BwdParams& p, int dtype, int d, bool causal, hipStream_t stream) {
  const bool bf = dtype == kDtypeBf16;
  if (d == 128) {
    if (bf) return causal ? launch_bwd_atomic_t<128, true, true>(p, stream) : launch_bwd_atomic_t<128, true, false>(p, stream);
    return causal ? launch_bwd_atomic_t<128, false, true>(p, stream) : launch_bwd_atomic_t<128, false, false>(p, stream);
  }
  if (bf) return causal ? launch_bwd_atomic_t<64, true, true>(p, stream) : launch_bwd_atomic_t<64, true, false>(p, stream);
  return causal ? launch_bwd_atomic_t<64, false, true>(p, stream) : launch_bwd_atomic_t<64, false, false>(p, stream);
}

hipError_t launch_bwd(const BwdParams& p, int dtype, int d, bool causal, hipStream_t stream) {
  if (dtype == kDtypeFp32) return launch_bwd32(p, d, causal, stream);
  const bool bf = dtype == kDtypeBf16;
  if (d == 128) return bf ? launch_bwd_c<128, true>(p, causal, stream) : launch_bwd_c<128, false>(p, causal, stream);
  return bf ? launch_bwd_c<64, true>(p, causal, stream) : launch_bwd_c<64, false>(p, causal, stream);
}

hipError_t launch_bwd_varlen(const BwdParams& p, int dtype, int d, bool causal, hipStream_t stream) {
  const bool bf = dtype == kDtypeBf16;
  if (d == 128) {
    if (bf) return causal ? launch_bwd_varlen_t<128, true, true>(p, stream) : launch_bwd_varlen_t<128, true, false>(p, stream);
    return causal ? launch_bwd_varlen_t<128, false, true>(p, stream) : launch_bwd_varlen_t<128, false, false>(p, stream);
  }
  if (bf) return causal ? launch_bwd_varlen_t<64, true, true>(p, stream) : launch_bwd_varlen_t<64, true, false>(p, stream);
  return causal ? launch_bwd_varlen_t<64, false, true>(p, stream) : launch_bwd_varlen_t<64, false, false>(p, stream);
}

int bwd_rows_per_workgroup() { return 128; }

}  // namespace fa
