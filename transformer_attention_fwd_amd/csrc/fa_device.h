// fa_device.h -- device-side building blocks shared by the attention kernels (gfx950 only, not installed):
// vector types, MFMA wrappers for the two 16-bit input types, wait-counter and barrier helpers, the
// buffer-load-to-LDS issue of a pair of tiles, and the workgroup -> (head, tile) order.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr float kLn2 = 0.693147180559945309f;
constexpr float kNegInf = -__builtin_inff();
// word 3 of a buffer resource on gfx9-family parts: 32-bit data format, raw (unswizzled) addressing
constexpr int kBufferFlags = 0x00020000;

// s_waitcnt immediate for "vmcnt <= n" on gfx9-family encodings (expcnt and lgkmcnt left free).
__device__ constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
// s_waitcnt immediate for "lgkmcnt == 0" (vmcnt and expcnt left free).
__device__ constexpr int waitcnt_lgkm0() { return 15 | (3 << 14) | (7 << 4); }

__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }
__device__ __forceinline__ void keep_branch() { asm volatile(""); }

// Workgroup barrier for LDS hand-offs: the caller has already waited for the loads it needs.
__device__ __forceinline__ void lds_barrier() {
  compiler_fence();
  __builtin_amdgcn_s_waitcnt(waitcnt_lgkm0());
  __builtin_amdgcn_s_barrier();
  compiler_fence();
}

// Block index -> (b*H + h, q_tile).  Workgroups reach the 8 XCDs round robin; XCD x gets a
// contiguous run of the head-major unit list, heaviest causal tiles first inside each head.
__device__ __forceinline__ void unit_of(int bid, int n_units, int n_qtiles, bool causal, int& bh, int& qt) {
  constexpr int X = 8;
  const int x = bid % X, u = bid / X;
  const int base = n_units / X, rem = n_units % X;
  const int L = x * base + (x < rem ? x : rem) + u;
  bh = L / n_qtiles;
  const int r = L - bh * n_qtiles;
  qt = causal ? n_qtiles - 1 - r : r;
}

// Block index -> (b*H + h, q_tile) spreading heads over the XCDs: XCD x (blocks x, x+8, ...) takes heads
// x, x+8, x+16, ... in turn, each head's tiles heaviest first when causal.  For work that differs from
// head to head (sequences of different lengths) this gives every XCD an equal share of each sequence.
// The grid covers ceil(BH/8)*8 heads; blocks that land on a padding head (bh >= BH) have no work.
__device__ __forceinline__ void unit_of_spread(int bid, int n_qtiles, bool causal, int& bh, int& qt) {
  constexpr int X = 8;
  const int x = bid % X, u = bid / X;
  const int m = u / n_qtiles, r = u - m * n_qtiles;
  bh = x + X * m;
  qt = causal ? n_qtiles - 1 - r : r;
}

__device__ __forceinline__ float wave_max_xor16_32(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}
__device__ __forceinline__ float wave_sum_xor16_32(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

template <bool IS_BF16>
struct Elem;
template <>
struct Elem<true> {
  typedef bf16x8_t vec8;
  __device__ static __forceinline__ uint32_t pack2(float a, float b) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    bf16x2_t v;
    v[0] = (__bf16)a;
    v[1] = (__bf16)b;
    return __builtin_bit_cast(uint32_t, v);
  }
  __device__ static __forceinline__ f32x4_t mfma(const vec8& a, const vec8& b, const f32x4_t& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  // all-ones operand: an MFMA against it sums the other operand's values as rounded
  __device__ static __forceinline__ vec8 ones() {
    const __bf16 o = (__bf16)1.0f;
    return vec8{o, o, o, o, o, o, o, o};
  }
};
template <>
struct Elem<false> {
  typedef f16x8_t vec8;
  __device__ static __forceinline__ uint32_t pack2(float a, float b) {
    typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
    f16x2_t v;
    v[0] = (_Float16)a;
    v[1] = (_Float16)b;
    return __builtin_bit_cast(uint32_t, v);
  }
  __device__ static __forceinline__ f32x4_t mfma(const vec8& a, const vec8& b, const f32x4_t& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ vec8 ones() {
    const _Float16 o = (_Float16)1.0f;
    return vec8{o, o, o, o, o, o, o, o};
  }
};

// Buffer loads of one K and one V tile straight into LDS: lane slot (i*NW + wave)*64 + lane of a tile
// holds the global 16-byte chunk at byte offset voff[i] + soff from the head base.
template <int LOADS, int NW>
__device__ __forceinline__ void issue_kv_tile(__amdgpu_buffer_rsrc_t kbuf, __amdgpu_buffer_rsrc_t vbuf,
                                              const int* voff_k, const int* voff_v, int soff, int wave,
                                              uint8_t* kdst, uint8_t* vdst) {
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int lds_off = (i * NW + wave) * 1024;  // wave-uniform base; lane lands at +16*lane
    __builtin_amdgcn_raw_ptr_buffer_load_lds(kbuf, (lds_void_t*)(kdst + lds_off), 16, voff_k[i], soff, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(vbuf, (lds_void_t*)(vdst + lds_off), 16, voff_v[i], soff, 0, 0);
  }
}

}  // namespace fa
