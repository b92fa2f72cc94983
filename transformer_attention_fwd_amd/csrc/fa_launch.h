// fa_launch.h -- internal interface between the C-ABI entry point and the kernels (not installed).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

constexpr int kDtypeFp32 = 0;
constexpr int kDtypeFp16 = 1;
constexpr int kDtypeBf16 = 2;

// Kernel arguments.  Strides are in elements; the (b, h) base of a tensor is b*stride_b + h*stride_h
// and consecutive sequence positions are stride_s apart (D for [B][H][N][D], H*D for [B][N][H][D]).
struct Params {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int64_t stride_b;
  int64_t stride_h;
  int64_t stride_s;
  int B, H, N;
  int n_qtiles;   // filled by the launcher
  int n_units;    // filled by the launcher
  float c;        // |scale| * log2(e), > 0 (a zero scale is passed as FLT_MIN by the entry point)
  uint32_t qsign; // XOR mask applied to Q's stored bits: flips the sign when scale < 0
};

// Enqueue the kernel for (dtype, d, causal) on `stream`.
hipError_t launch(const Params& p, int dtype, int d, bool causal, hipStream_t stream);

// Queries handled by one workgroup for a dtype (for callers that size grids or count work).
int queries_per_workgroup(int dtype);

}  // namespace fa
