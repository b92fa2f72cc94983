// fa_bwd32.hip -- attention backward kernels for gfx950 (MI355X, CDNA4), fp32 inputs.
//
// The same gradients as the 16-bit kernels, fp32 end to end:
//     dV = P^T dO,   dP = dO V^T,   D_i = sum_d dO_id O_id,   dS = P o (dP - D),
//     dQ = scale * dS K,   dK = scale * dS^T Q,
// with P recomputed from the forward's lse as exp(scale * q.k - lse) (page ai6s.net/6a0d3bfb..., section
// "FlashAttention在昇腾NPU上怎么跑？", item 3: the backward recomputes instead of storing N x N
// matrices).  Deterministic (no atomics), the same two-kernel split, visibility rule and key chunk as
// the 16-bit path:
//   fa_bwd_dq32   one workgroup per (b, h, 128-query tile), 4 waves x 32 queries; K/V tiles of 32 keys
//                 staged in LDS.  Per tile S^T = K Q^T, dP^T = V dO^T, dS^T, then dQ^T += K^T dS^T.
//   fa_bwd_dkdv32 one workgroup per (b, h, 128-key tile), 4 waves x 32 keys kept in registers; Q/dO
//                 tiles of 32 rows staged in LDS with their rows' lse and D.  Per tile S = Q K^T,
//                 dP = dO V^T, P, dS, then dV^T += dO^T P and dK^T += Q^T dS.
// MFMA v_mfma_f32_16x16x4_f32: A is one float per lane (row lane % 16, k lane / 16), B one float per
// lane (column lane % 16, k lane / 16), and the 16x16 C tile holds rows 4 (lane / 16) + r, column
// lane % 16 in a lane's four registers -- so a C tile is a B operand k step by step: for fixed r, lane
// (column c, group g) holds C[4 g + r][c], i.e. B[k = g][c] of the product over rows 4 g + r.
// Visibility is tested per element on 64-bit positions: query row i sits at q_offset + i, key j at j.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_device.h"
#include "fa_bwd_launch.h"

namespace fa {
namespace {

constexpr float kLog2e32 = 1.44269504088896341f;

template <int D>
struct Bwd32Tile {
  static constexpr int NW = 4;        // waves per workgroup
  static constexpr int RW = 32;       // rows (queries or keys) per wave
  static constexpr int BM = NW * RW;  // rows per workgroup (128: the grid tile of both kernels)
  static constexpr int BT = 32;       // rows of a streamed tile (K/V in dQ, Q/dO in dK/dV)
  static constexpr int RG = RW / 16;  // 16-row groups per wave
  static constexpr int TG = BT / 16;  // 16-row groups per streamed tile
  static constexpr int DK = D / 4;    // k steps of the products over d
  static constexpr int DT = D / 16;   // 16-wide d tiles of dQ^T, dK^T, dV^T
  static constexpr int LD = D + 4;    // padded LDS row (floats): rows 4 apart start 16 banks apart
};

__device__ __forceinline__ f32x4_t mfma32(float a, float b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// key j visible to the query at position qpos (inside the chunk [kv0, kv1))
template <bool CAUSAL, bool WINDOW>
__device__ __forceinline__ bool visible32(int64_t key, int64_t qpos, int kv0, int kv1, int64_t window) {
  return key >= kv0 && key < kv1 && (!CAUSAL || key <= qpos) && (!WINDOW || key >= qpos - window);
}

template <int D, bool CAUSAL, bool WINDOW>
__global__ __launch_bounds__(256, 1) void fa_bwd_dq32(BwdParams p) {
  typedef Bwd32Tile<D> T;
  __shared__ float ks[T::BT * T::LD];
  __shared__ float vs[T::BT * T::LD];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4, li = lane & 15;
  int bh, qt;
  unit_of(blockIdx.x, p.n_units_q, p.n_tiles_q, CAUSAL, bh, qt);
  const int b = bh / p.H, h = bh - (bh / p.H) * p.H;
  const int Nq = p.Nq;
  const int64_t qoff = p.q_offset, window = p.window;
  const int kv0 = p.kv_start, kv1 = p.kv_start + p.kv_len;
  const int q_wg = qt * T::BM, q0 = q_wg + wave * T::RW;
  const int64_t qhead = b * p.stride_b_q + h * p.stride_h_q;
  const int64_t khead = b * p.stride_b_k + h * p.stride_h_k;
  const int64_t ss = p.stride_s;
  const float* qp = (const float*)p.q + qhead;
  const float* op = (const float*)p.o + qhead;
  const float* dop = (const float*)p.dout + qhead;
  const float* kp = (const float*)p.k + khead;
  const float* vp = (const float*)p.v + khead;

  // Q^T and dO^T as B operands: lane holds row q0 + 16*qg + li, d = 4*kk + g.  D_i from the same
  // pattern of O, summed over the four lane groups.
  float qf[T::RG][T::DK], df[T::RG][T::DK];
  float lse2[T::RG], dlt[T::RG];
#pragma unroll
  for (int qg = 0; qg < T::RG; ++qg) {
    const int qi = q0 + 16 * qg + li;
    const int qrow = min(qi, Nq - 1);
    float acc = 0.f;
#pragma unroll
    for (int kk = 0; kk < T::DK; ++kk) {
      const int64_t e = qrow * ss + 4 * kk + g;
      qf[qg][kk] = qp[e];
      df[qg][kk] = dop[e];
      acc = __builtin_fmaf(df[qg][kk], op[e], acc);
    }
    dlt[qg] = wave_sum_xor16_32(acc);
    lse2[qg] = p.lse[(int64_t)bh * Nq + qrow] * kLog2e32;
    if (g == 0 && qi < Nq) p.delta[(int64_t)bh * Nq + qi] = dlt[qg];
  }

  // the chunk's keys that some query of this workgroup sees
  const int k_lo = WINDOW ? (int)max((int64_t)kv0, q_wg + qoff - window) : kv0;
  const int k_hi = CAUSAL ? (int)min((int64_t)kv1 - 1, q_wg + T::BM - 1 + qoff) : kv1 - 1;
  const int n_kt = k_hi >= k_lo ? (k_hi - k_lo) / T::BT + 1 : 0;
  const float cexp = p.c;
  f32x4_t dqa[T::RG][T::DT];
#pragma unroll
  for (int qg = 0; qg < T::RG; ++qg)
#pragma unroll
    for (int dt = 0; dt < T::DT; ++dt) dqa[qg][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int j = 0; j < n_kt; ++j) {
    const int key0 = k_lo + j * T::BT;
    // stage the K and V rows of the tile (rows past the chunk repeat its last row and are hidden)
    for (int idx = threadIdx.x; idx < T::BT * (D / 4); idx += 64 * T::NW) {
      const int row = idx / (D / 4), c4 = idx % (D / 4);
      const int key = min(key0 + row, kv1 - 1);
      *(float4*)(ks + row * T::LD + 4 * c4) = *(const float4*)(kp + key * ss + 4 * c4);
      *(float4*)(vs + row * T::LD + 4 * c4) = *(const float4*)(vp + key * ss + 4 * c4);
    }
    __syncthreads();
    // some query of the wave sees some key of the tile
    const bool active = (!CAUSAL || key0 <= q0 + T::RW - 1 + qoff) && (!WINDOW || key0 + T::BT - 1 >= q0 + qoff - window);
    if (active) {
      // S^T and dP^T: lane holds keys key0 + 16*kt + 4*g + r for query q0 + 16*qg + li
      f32x4_t s[T::RG][T::TG], dp[T::RG][T::TG];
#pragma unroll
      for (int kt = 0; kt < T::TG; ++kt) {
#pragma unroll
        for (int qg = 0; qg < T::RG; ++qg) {
          s[qg][kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
          dp[qg][kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int kk = 0; kk < T::DK; ++kk) {
          const float kf = ks[(16 * kt + li) * T::LD + 4 * kk + g];
          const float vf = vs[(16 * kt + li) * T::LD + 4 * kk + g];
#pragma unroll
          for (int qg = 0; qg < T::RG; ++qg) {
            s[qg][kt] = mfma32(kf, qf[qg][kk], s[qg][kt]);
            dp[qg][kt] = mfma32(vf, df[qg][kk], dp[qg][kt]);
          }
        }
      }
      // dS = P o (dP - D), P = 0 where the key is hidden
#pragma unroll
      for (int qg = 0; qg < T::RG; ++qg) {
        const int64_t qpos = (int64_t)(q0 + 16 * qg + li) + qoff;
#pragma unroll
        for (int kt = 0; kt < T::TG; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = key0 + 16 * kt + 4 * g + r;
            const float pr = visible32<CAUSAL, WINDOW>(key, qpos, kv0, kv1, window)
                                 ? __builtin_amdgcn_exp2f(__builtin_fmaf(s[qg][kt][r], cexp, -lse2[qg]))
                                 : 0.f;
            s[qg][kt][r] = pr * (dp[qg][kt][r] - dlt[qg]);
          }
      }
      // dQ^T += K^T dS^T, one k step per (kt, r): key slot g <-> key 16*kt + 4*g + r
#pragma unroll
      for (int kt = 0; kt < T::TG; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int dt = 0; dt < T::DT; ++dt) {
            const float kf = ks[(16 * kt + 4 * g + r) * T::LD + 16 * dt + li];
#pragma unroll
            for (int qg = 0; qg < T::RG; ++qg) dqa[qg][dt] = mfma32(kf, s[qg][kt][r], dqa[qg][dt]);
          }
    }
    __syncthreads();
  }

  // dQ: lane holds d = 16*dt + 4*g .. +3 of query q0 + 16*qg + li
  float* dqp = (float*)p.dq + qhead;
#pragma unroll
  for (int qg = 0; qg < T::RG; ++qg) {
    const int qi = q0 + 16 * qg + li;
    if (qi < Nq) {
#pragma unroll
      for (int dt = 0; dt < T::DT; ++dt) {
        const f32x4_t x = dqa[qg][dt] * p.scale;
        *(float4*)(dqp + qi * ss + 16 * dt + 4 * g) = make_float4(x[0], x[1], x[2], x[3]);
      }
    }
  }
}

template <int D, bool CAUSAL, bool WINDOW>
__global__ __launch_bounds__(256, 1) void fa_bwd_dkdv32(BwdParams p) {
  typedef Bwd32Tile<D> T;
  __shared__ float qs[T::BT * T::LD];
  __shared__ float os[T::BT * T::LD];
  __shared__ float rl[T::BT];  // lse * log2(e) of the tile's rows (+inf past Nq: P = 0)
  __shared__ float rd[T::BT];  // D of the tile's rows

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4, li = lane & 15;
  int bh, kt;
  unit_of(blockIdx.x, p.n_units_k, p.n_tiles_k, false, bh, kt);
  const int b = bh / p.H, h = bh - (bh / p.H) * p.H;
  const int Nq = p.Nq;
  const int64_t qoff = p.q_offset, window = p.window;
  const int kv0 = p.kv_start, kv1 = p.kv_start + p.kv_len;
  const int k_wg = kv0 + kt * T::BM, kw0 = k_wg + wave * T::RW;
  const int64_t qhead = b * p.stride_b_q + h * p.stride_h_q;
  const int64_t khead = b * p.stride_b_k + h * p.stride_h_k;
  const int64_t ss = p.stride_s;
  const float* qp = (const float*)p.q + qhead;
  const float* dop = (const float*)p.dout + qhead;
  const float* kp = (const float*)p.k + khead;
  const float* vp = (const float*)p.v + khead;

  // K^T and V^T as B operands of S = Q K^T and dP = dO V^T: lane holds key kw0 + 16*kg + li, d = 4*kk + g
  // (keys past the chunk repeat its last key and are hidden)
  float kf[T::RG][T::DK], vf[T::RG][T::DK];
#pragma unroll
  for (int kg = 0; kg < T::RG; ++kg) {
    const int krow = min(kw0 + 16 * kg + li, kv1 - 1);
#pragma unroll
    for (int kk = 0; kk < T::DK; ++kk) {
      kf[kg][kk] = kp[krow * ss + 4 * kk + g];
      vf[kg][kk] = vp[krow * ss + 4 * kk + g];
    }
  }
  f32x4_t dka[T::RG][T::DT], dva[T::RG][T::DT];
#pragma unroll
  for (int kg = 0; kg < T::RG; ++kg)
#pragma unroll
    for (int dt = 0; dt < T::DT; ++dt) {
      dka[kg][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      dva[kg][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

  // the query rows that see some key of this workgroup
  const int i_begin = CAUSAL ? (int)min((int64_t)Nq, max((int64_t)0, k_wg - qoff)) : 0;
  const int i_last = WINDOW ? (int)min((int64_t)Nq - 1, k_wg + T::BM - 1 + window - qoff) : Nq - 1;
  const int n_qt = i_last >= i_begin ? (i_last - i_begin) / T::BT + 1 : 0;
  const float cexp = p.c;

  for (int jt = 0; jt < n_qt; ++jt) {
    const int qb = i_begin + jt * T::BT;
    // stage the Q and dO rows of the tile and their lse * log2(e) and D
    for (int idx = threadIdx.x; idx < T::BT * (D / 4); idx += 64 * T::NW) {
      const int row = idx / (D / 4), c4 = idx % (D / 4);
      const int qrow = min(qb + row, Nq - 1);
      *(float4*)(qs + row * T::LD + 4 * c4) = *(const float4*)(qp + qrow * ss + 4 * c4);
      *(float4*)(os + row * T::LD + 4 * c4) = *(const float4*)(dop + qrow * ss + 4 * c4);
    }
    if (threadIdx.x < T::BT) {
      const int qi = qb + threadIdx.x;
      rl[threadIdx.x] = qi < Nq ? p.lse[(int64_t)bh * Nq + qi] * kLog2e32 : __builtin_inff();
      rd[threadIdx.x] = qi < Nq ? p.delta[(int64_t)bh * Nq + qi] : 0.f;
    }
    __syncthreads();
    // some query of the tile sees some key of the wave
    const bool active = (!CAUSAL || qb + T::BT - 1 + qoff >= kw0) && (!WINDOW || qb + qoff <= kw0 + T::RW - 1 + window);
    if (active) {
#pragma unroll 1
      for (int qq = 0; qq < T::TG; ++qq) {
        // S and dP: lane holds queries qb + 16*qq + 4*g + r for key kw0 + 16*kg + li
        f32x4_t s[T::RG], dp[T::RG];
#pragma unroll
        for (int kg = 0; kg < T::RG; ++kg) {
          s[kg] = f32x4_t{0.f, 0.f, 0.f, 0.f};
          dp[kg] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int kk = 0; kk < T::DK; ++kk) {
          const float qa = qs[(16 * qq + li) * T::LD + 4 * kk + g];
          const float oa = os[(16 * qq + li) * T::LD + 4 * kk + g];
#pragma unroll
          for (int kg = 0; kg < T::RG; ++kg) {
            s[kg] = mfma32(qa, kf[kg][kk], s[kg]);
            dp[kg] = mfma32(oa, vf[kg][kk], dp[kg]);
          }
        }
        // P and dS = P o (dP - D); P = 0 where the key is hidden or the row lies past Nq
        f32x4_t pr[T::RG], ds[T::RG];
#pragma unroll
        for (int kg = 0; kg < T::RG; ++kg) {
          const int key = kw0 + 16 * kg + li;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = 16 * qq + 4 * g + r;
            const int64_t qpos = (int64_t)(qb + row) + qoff;
            const float pv = (qb + row < Nq && visible32<CAUSAL, WINDOW>(key, qpos, kv0, kv1, window))
                                 ? __builtin_amdgcn_exp2f(__builtin_fmaf(s[kg][r], cexp, -rl[row]))
                                 : 0.f;
            pr[kg][r] = pv;
            ds[kg][r] = pv * (dp[kg][r] - rd[row]);
          }
        }
        // dV^T += dO^T P and dK^T += Q^T dS, one k step per r: query slot g <-> row 16*qq + 4*g + r
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int dt = 0; dt < T::DT; ++dt) {
            const float oa = os[(16 * qq + 4 * g + r) * T::LD + 16 * dt + li];
            const float qa = qs[(16 * qq + 4 * g + r) * T::LD + 16 * dt + li];
#pragma unroll
            for (int kg = 0; kg < T::RG; ++kg) {
              dva[kg][dt] = mfma32(oa, pr[kg][r], dva[kg][dt]);
              dka[kg][dt] = mfma32(qa, ds[kg][r], dka[kg][dt]);
            }
          }
      }
    }
    __syncthreads();
  }

  // dK, dV of the chunk's keys: lane holds d = 16*dt + 4*g .. +3 of key kw0 + 16*kg + li
  float* dkp = (float*)p.dk + khead;
  float* dvp = (float*)p.dv + khead;
#pragma unroll
  for (int kg = 0; kg < T::RG; ++kg) {
    const int key = kw0 + 16 * kg + li;
    if (key < kv1) {
#pragma unroll
      for (int dt = 0; dt < T::DT; ++dt) {
        const f32x4_t x = dka[kg][dt] * p.scale;
        const f32x4_t y = dva[kg][dt];
        *(float4*)(dkp + key * ss + 16 * dt + 4 * g) = make_float4(x[0], x[1], x[2], x[3]);
        *(float4*)(dvp + key * ss + 16 * dt + 4 * g) = make_float4(y[0], y[1], y[2], y[3]);
      }
    }
  }
}

template <int D, bool CAUSAL, bool WINDOW>
hipError_t launch_bwd32_t(BwdParams p, hipStream_t stream) {
  typedef Bwd32Tile<D> T;
  p.n_tiles_q = (p.Nq + T::BM - 1) / T::BM;
  p.n_units_q = p.B * p.H * p.n_tiles_q;
  p.n_tiles_k = (p.kv_len + T::BM - 1) / T::BM;
  p.n_units_k = p.B * p.H * p.n_tiles_k;
  hipLaunchKernelGGL((fa_bwd_dq32<D, CAUSAL, WINDOW>), dim3(p.n_units_q), dim3(64 * T::NW), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.n_units_k == 0) return e;
  hipLaunchKernelGGL((fa_bwd_dkdv32<D, CAUSAL, WINDOW>), dim3(p.n_units_k), dim3(64 * T::NW), 0, stream, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_bwd32_c(const BwdParams& p, bool causal, hipStream_t stream) {
  if (!causal) return launch_bwd32_t<D, false, false>(p, stream);
  return p.window >= 0 ? launch_bwd32_t<D, true, true>(p, stream) : launch_bwd32_t<D, true, false>(p, stream);
}

}  // namespace

hipError_t launch_bwd32(const BwdParams& p, int d, bool causal, hipStream_t stream) {
  return d == 128 ? launch_bwd32_c<128>(p, causal, stream) : launch_bwd32_c<64>(p, causal, stream);
}

}  // namespace fa
