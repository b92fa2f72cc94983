// fa_merge.hip -- combination of partial attention results over disjoint key sets.
//
// A long key sequence processed in chunks (ring / block-wise attention: page ai6s.net/6a0d3bfb...,
// section "ops-transformer仓库里还有什么？"; a 64K sequence split into 8K pieces: page ai6s.net/6a140d07...,
// section "多卡并行") gives one (O_s, lse_s) per chunk.  They combine exactly through the log-sum-exp,
// shifted by the largest one (same page, section "第二层：数值稳定性增强"):
//     M = max_s lse_s,  w_s = exp(lse_s - M),  lse = M + ln sum_s w_s,  O = sum_s (w_s / sum_s w_s) O_s.
// A part with lse_s = -inf (no visible key) has weight 0; a row where every part has -inf gets O = 0,
// lse = -inf.
//
// Memory-bound: every part's O row and lse are read once and the result written once.  One thread
// combines 8 consecutive elements of one row (16-byte loads for 16-bit types, two for fp32), in fp32.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_launch.h"

namespace fa {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
constexpr float kLog2e = 1.44269504088896341f;
constexpr float kLn2m = 0.693147180559945309f;

// 8 stored elements <-> fp32
template <int DT>
struct Pack8;
template <>
struct Pack8<kDtypeFp32> {
  __device__ static void load(const void* base, int64_t e, float* x) {
    const float4 a = *(const float4*)((const float*)base + e);
    const float4 b = *(const float4*)((const float*)base + e + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
  __device__ static void store(void* base, int64_t e, const float* x) {
    *(float4*)((float*)base + e) = make_float4(x[0], x[1], x[2], x[3]);
    *(float4*)((float*)base + e + 4) = make_float4(x[4], x[5], x[6], x[7]);
  }
};
template <>
struct Pack8<kDtypeBf16> {
  __device__ static void load(const void* base, int64_t e, float* x) {
    const u32x4_t w = *(const u32x4_t*)((const uint16_t*)base + e);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  __device__ static void store(void* base, int64_t e, const float* x) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    u32x4_t w;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bf16x2_t v;
      v[0] = (__bf16)x[2 * i];
      v[1] = (__bf16)x[2 * i + 1];
      w[i] = __builtin_bit_cast(uint32_t, v);
    }
    *(u32x4_t*)((uint16_t*)base + e) = w;
  }
};
template <>
struct Pack8<kDtypeFp16> {
  __device__ static void load(const void* base, int64_t e, float* x) {
    typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
    const f16x8_t w = *(const f16x8_t*)((const uint16_t*)base + e);
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = (float)w[i];
  }
  __device__ static void store(void* base, int64_t e, const float* x) {
    typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
    f16x8_t w;
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = (_Float16)x[i];
    *(f16x8_t*)((uint16_t*)base + e) = w;
  }
};

// Thread t: lse row r = t / (D/8) in [B][H][N] order, elements 8*(t % (D/8)) .. +7 of that row.
template <int DT, int D>
__global__ __launch_bounds__(256) void fa_merge_kernel(const void* __restrict__ o_parts, const float* __restrict__ lse_parts,
                                                       int n_parts, void* __restrict__ o, float* __restrict__ lse,
                                                       int64_t rows, int64_t H, int64_t N, int bsnd) {
  constexpr int TPR = D / 8;  // threads per row
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t r = t / TPR;
  if (r >= rows) return;
  const int c = (int)(t - r * TPR);
  // element offset of the row in the layout
  int64_t orow = r;
  if (bsnd) {
    const int64_t i = r % N, bh = r / N, h = bh % H, b = bh / H;
    orow = (b * N + i) * H + h;
  }
  const int64_t e = orow * D + 8 * c;
  const int64_t part_elems = rows * D;

  float m = -__builtin_inff();
  for (int s = 0; s < n_parts; ++s) m = fmaxf(m, lse_parts[s * rows + r]);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float out_lse = -__builtin_inff();
  if (m != -__builtin_inff()) {
    float tot = 0.f;
    // parts in groups of U whose loads are in flight together, summed in part order; a part without
    // visible keys (or whose weight underflows to 0) is not loaded and adds exactly nothing
    constexpr int U = 4;
    for (int s0 = 0; s0 < n_parts; s0 += U) {
      float w[U], x[U][8];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int s = s0 + u;
        const float ls = s < n_parts ? lse_parts[s * rows + r] : -__builtin_inff();
        w[u] = ls == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f((ls - m) * kLog2e);
        if (w[u] != 0.f) {
          Pack8<DT>::load(o_parts, s * part_elems + e, x[u]);
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) x[u][i] = 0.f;
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        tot += w[u];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = __builtin_fmaf(w[u], x[u][i], acc[i]);
      }
    }
    const float inv = 1.0f / tot;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] *= inv;
    out_lse = m + __builtin_amdgcn_logf(tot) * kLn2m;
  }
  Pack8<DT>::store(o, e, acc);
  if (c == 0) lse[r] = out_lse;
}

}  // namespace

hipError_t launch_merge(const void* o_parts, const float* lse_parts, int n_parts, void* o, float* lse, int64_t rows,
                        int64_t B, int64_t H, int64_t N, int D, int layout_bsnd, int dtype, hipStream_t stream) {
  (void)B;
  const int64_t threads = rows * (D / 8);
  const dim3 grid((unsigned)((threads + 255) / 256)), block(256);
#define FA_MERGE_LAUNCH(DT, DD) \
  hipLaunchKernelGGL((fa_merge_kernel<DT, DD>), grid, block, 0, stream, o_parts, lse_parts, n_parts, o, lse, rows, H, N, layout_bsnd)
  if (dtype == kDtypeBf16) {
    if (D == 128) FA_MERGE_LAUNCH(kDtypeBf16, 128); else FA_MERGE_LAUNCH(kDtypeBf16, 64);
  } else if (dtype == kDtypeFp16) {
    if (D == 128) FA_MERGE_LAUNCH(kDtypeFp16, 128); else FA_MERGE_LAUNCH(kDtypeFp16, 64);
  } else {
    if (D == 128) FA_MERGE_LAUNCH(kDtypeFp32, 128); else FA_MERGE_LAUNCH(kDtypeFp32, 64);
  }
#undef FA_MERGE_LAUNCH
  return hipGetLastError();
}

}  // namespace fa
