// fa_launch.h -- internal interface between the C-ABI entry point and the forward and merge kernels
// (not installed).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

constexpr int kDtypeFp32 = 0;
constexpr int kDtypeFp16 = 1;
constexpr int kDtypeBf16 = 2;

// Kernel arguments.  Strides are in elements.  The (b, h) base of Q and O is b*stride_b_q + h*stride_h_q,
// that of K and V b*stride_b_k + h*stride_h_k + kv_start*stride_s; consecutive sequence positions are
// stride_s apart in all four (D for [B][H][rows][D], H*D for [B][rows][H][D]).
// Query row i sits at sequence position q_offset + i and key row j of the chunk at kv_start + j, so key
// j is causally visible to query i iff j <= i + delta with delta = q_offset - kv_start, and inside the
// window iff j >= i + delta - window.
struct Params {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;       // [B][H][Nq]
  int64_t stride_b_q, stride_h_q;
  int64_t stride_b_k, stride_h_k;
  int64_t stride_s;
  int64_t kv_start;
  int B, H;
  int Nq;           // query rows
  int Nkv;          // keys in the chunk (may be 0)
  int64_t delta;    // q_offset - kv_start
  int64_t window;   // keys before the query's position that stay visible; < 0: no window
  int n_qtiles;     // filled by the launcher
  int n_units;      // filled by the launcher
  float c;          // |scale| * log2(e), > 0 (a zero scale is passed as FLT_MIN by the entry point)
  uint32_t qsign;   // XOR mask applied to Q's stored bits: flips the sign when scale < 0
  // Packed variable-length batches only (null otherwise): sequence b owns query rows cu_q[b] ..
  // cu_q[b+1]-1 of the [total_q][H][D] tensors and key rows cu_k[b] .. cu_k[b+1]-1 of [total_k][H][D];
  // Nq then holds the longest query count (grid sizing) and lse is [H][total_q].
  const int* cu_q;
  const int* cu_k;
  int64_t total_q, total_k;
  // Set by the launcher when it splits a call into launches over row ranges (0 from the entry points):
  // this launch computes rows q_row0 .. q_row0 + Nq - 1 of each head, whose lse rows hold lse_rows
  // entries (0: Nq); rec_base is its first tile-record slot (test builds).
  int q_row0;
  int64_t lse_rows;
  int rec_base;
  // A key chunk split into row ranges in one launch of the ping-pong kernel: rows 0 .. Nkv - 1 (from
  // q_row0) are its square, the n_rect * 256 rows after it see every key (run in chains of n_chain units
  // per block), and the n_empty rows before q_row0 see none.
  int n_rect, n_empty, n_chain;
};

// Enqueue the attention kernel for (dtype, d, causal, window >= 0) on `stream`.
hipError_t launch(const Params& p, int dtype, int d, bool causal, hipStream_t stream);

// Enqueue the packed variable-length forward (16-bit dtypes; Params::cu_q / cu_k set) on `stream`.
hipError_t launch_varlen(const Params& p, int dtype, int d, bool causal, hipStream_t stream);

// Enqueue the combination of n_parts partial results (see fa_merge in fa.h).
hipError_t launch_merge(const void* o_parts, const float* lse_parts, int n_parts, void* o, float* lse, int64_t rows,
                        int64_t B, int64_t H, int64_t N, int D, int layout_bsnd, int dtype, hipStream_t stream);

// Queries handled by one workgroup for a dtype (for callers that size grids or count work).
int queries_per_workgroup(int dtype);

}  // namespace fa
