// fa_bwd_launch.h -- internal interface between the C-ABI entry point and the backward kernels (not
// installed).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_launch.h"

namespace fa {

// Backward kernel arguments.  Query row i sits at position q_offset + i and key row j at j; key j is
// visible to query i iff (causal) j <= q_offset + i and (window >= 0) j >= q_offset + i - window.  The
// key chunk [kv_start, kv_start + kv_len) bounds the keys dQ sums over and the dK/dV rows written.
// Q, O, dO, dQ rows: base b*stride_b_q + h*stride_h_q; K, V, dK, dV: b*stride_b_k + h*stride_h_k;
// consecutive rows stride_s apart (elements).
struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;   // [B][H][Nq], natural log, of the forward over every visible key
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* delta;       // [B][H][Nq] workspace: D_i = sum_d dO_id O_id, written by the dQ kernel
  float* dq_acc;      // atomic mode only: fp32 dQ accumulator laid out like dq (null otherwise)
  int64_t stride_b_q, stride_h_q, stride_b_k, stride_h_k, stride_s;
  int64_t q_offset;
  int64_t window;     // < 0: no window
  int B, H, Nq, Nk;
  int kv_start, kv_len;
  int n_tiles_q, n_units_q;  // filled by the launcher
  int n_tiles_k, n_units_k;  // filled by the launcher
  float c;            // scale * log2(e), signed
  float scale;
  // Packed variable-length batches only (null otherwise): sequence b owns query rows cu_q[b] ..
  // cu_q[b+1]-1 of the [total_q][H][D] tensors and key rows cu_k[b] .. cu_k[b+1]-1 of [total_k][H][D];
  // Nq and Nk then hold the longest query and key counts (grid sizing) and lse, delta are [H][total_q].
  const int* cu_q;
  const int* cu_k;
  int64_t total_q, total_k;
};

// Enqueue the two backward kernels (dQ and D, then dK and dV) for `dtype` on `stream`; a window is used
// only with causal.
hipError_t launch_bwd(const BwdParams& p, int dtype, int d, bool causal, hipStream_t stream);

// Enqueue the backward of packed variable-length batches (16-bit dtypes; BwdParams::cu_q / cu_k set).
hipError_t launch_bwd_varlen(const BwdParams& p, int dtype, int d, bool causal, hipStream_t stream);

// Enqueue the atomic mode (16-bit dtypes, no window, no key chunk): D and a zeroed p.dq_acc, then the dK/dV
// kernel that also adds dQ's parts into p.dq_acc with atomics, then dq = scale * dq_acc rounded to dtype.
hipError_t launch_bwd_atomic(const BwdParams& p, int dtype, int d, bool causal, hipStream_t stream);

// The fp32 kernels behind launch_bwd.
hipError_t launch_bwd32(const BwdParams& p, int d, bool causal, hipStream_t stream);

// Query (and key) rows handled by one backward workgroup.
int bwd_rows_per_workgroup();

}  // namespace fa
