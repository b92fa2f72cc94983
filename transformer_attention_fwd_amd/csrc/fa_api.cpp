// fa_api.cpp -- the C-ABI entry point of libfa.so: argument checks, device-residency checks, dispatch.
//
// Pure argument checks come first and touch no HIP API, so they behave the same on a host without a
// GPU.  The error conventions answer the deployment page's error table (hwcomputing.csdn.net/
// 6a0d4444..., section on common errors: host tensors crashing the operator, wrong input layout,
// head-count mismatch): every bad call returns a status code and launches nothing.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "../../include/fa.h"
#include "fa_bwd_launch.h"

#define FA_API extern "C" __attribute__((visibility("default")))

namespace {

thread_local char g_last_error[256] = "";

void set_error(const char* what, hipError_t e) {
  snprintf(g_last_error, sizeof g_last_error, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

bool mul_ok(int64_t a, int64_t b, int64_t* out) { return !__builtin_mul_overflow(a, b, out); }

// longest query or key sequence (and largest |q_offset|) accepted
constexpr int64_t kMaxRows = int64_t(1) << 30;

bool overlaps(const void* a, int64_t abytes, const void* b, int64_t bbytes) {
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + (uintptr_t)bbytes && b0 < a0 + (uintptr_t)abytes;
}

// Device memory of the current device (plain device allocation or managed memory).
int check_device(const void* ptr, int device) {
  hipPointerAttribute_t attr;
  memset(&attr, 0, sizeof attr);
  hipError_t e = hipPointerGetAttributes(&attr, ptr);
  if (e != hipSuccess) {
    (void)hipGetLastError();  // clear the sticky "invalid value" a host pointer can leave
    return FA_ERR_NOT_DEVICE_MEMORY;
  }
  if (attr.type != hipMemoryTypeDevice && attr.type != hipMemoryTypeManaged) return FA_ERR_NOT_DEVICE_MEMORY;
  if (attr.device != device) return FA_ERR_NOT_DEVICE_MEMORY;
  return FA_OK;
}

// The D workspace of fa_bwd_noalloc: one array per GPU, held until the process ends.  Every call on a GPU
// shares it (D is written by the backward's first kernel before its second reads it, so nothing needs
// clearing); calls that overlap on one GPU race on it.
constexpr int64_t kNoAllocMaxRows = FA_NOALLOC_MAX_ROWS;
__device__ __align__(256) float scratch[kNoAllocMaxRows];

// Device address of `scratch` on each device, looked up once per device (with that device current) by
// hipGetSymbolAddress: in host code the array's name is a host-side stand-in, never a device address.
constexpr int kMaxDevices = 64;
float* g_scratch_ptr[kMaxDevices] = {};
std::mutex g_scratch_mutex;

int scratch_of_device(int device, float** out) {
  if (device < 0 || device >= kMaxDevices) return FA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[device] == nullptr) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) {
      set_error("hipGetSymbolAddress(scratch)", e);
      return FA_ERR_HIP;
    }
    g_scratch_ptr[device] = (float*)ptr;
  }
  *out = g_scratch_ptr[device];
  return FA_OK;
}

}  // namespace

FA_API const char* fa_status_str(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "null pointer";
    case FA_ERR_BAD_DIM: return "B, H, N and D must be >= 1";
    case FA_ERR_BAD_LAYOUT: return "layout must be FA_LAYOUT_BHSD or FA_LAYOUT_BSND";
    case FA_ERR_BAD_DTYPE: return "dtype must be FA_DTYPE_FP32, FA_DTYPE_FP16 or FA_DTYPE_BF16";
    case FA_ERR_UNSUPPORTED: return "unsupported size: D must be 64 or 128, N <= 2^30, B*H < 2^31";
    case FA_ERR_BAD_SCALE: return "scale must be finite";
    case FA_ERR_MISALIGNED: return "tensor base pointers must be 16-byte aligned";
    case FA_ERR_ALIAS: return "o and lse must not overlap the inputs or each other";
    case FA_ERR_NOT_DEVICE_MEMORY: return "a pointer is not device memory of the current device";
    case FA_ERR_HIP: return "HIP runtime error";
    case FA_ERR_BAD_RANGE: return "key chunk outside [0, Nk], window without causal, q_offset out of range, or max_seqlen_q > total_q";
    case FA_ERR_SCRATCH_LIMIT: return "fa_bwd_noalloc: B*H*N exceeds the scratch array (FA_NOALLOC_MAX_ROWS rows)";
    default: return "unknown status";
  }
}

FA_API const char* fa_last_error(void) { return g_last_error; }

FA_API int fa_version(void) { return 600; }  // 0.6.0

FA_API int fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
                     int64_t Nq, int64_t Nk, int64_t D, int layout, int causal, int64_t window, int64_t q_offset,
                     int64_t kv_start, int64_t kv_len, float scale, int dtype, void* stream) {
  // ---- pure argument checks (no HIP calls) ----
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (layout != FA_LAYOUT_BHSD && layout != FA_LAYOUT_BSND) return FA_ERR_BAD_LAYOUT;
  if (dtype != FA_DTYPE_FP32 && dtype != FA_DTYPE_FP16 && dtype != FA_DTYPE_BF16) return FA_ERR_BAD_DTYPE;
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || D < 1) return FA_ERR_BAD_DIM;
  if (D != 64 && D != 128) return FA_ERR_UNSUPPORTED;
  int64_t bh, rows_q, rows_k, elems_q, elems_k, bytes_q, bytes_k, lse_bytes;
  const int64_t esize = dtype == FA_DTYPE_FP32 ? 4 : 2;
  if (Nq > kMaxRows || Nk > kMaxRows || !mul_ok(B, H, &bh) || bh > INT32_MAX || !mul_ok(bh, Nq, &rows_q) ||
      !mul_ok(bh, Nk, &rows_k) || !mul_ok(rows_q, D, &elems_q) || !mul_ok(rows_k, D, &elems_k) ||
      !mul_ok(elems_q, esize, &bytes_q) || !mul_ok(elems_k, esize, &bytes_k) || !mul_ok(rows_q, 4, &lse_bytes))
    return FA_ERR_UNSUPPORTED;
  if (kv_start < 0 || kv_len < 0 || kv_start > Nk || kv_len > Nk - kv_start) return FA_ERR_BAD_RANGE;
  if (window >= 0 && !causal) return FA_ERR_BAD_RANGE;
  if (q_offset < -kMaxRows || q_offset > kMaxRows) return FA_ERR_BAD_RANGE;
  // grid: one workgroup per (b, h, query tile); must fit a 32-bit grid dimension
  const int64_t qpw = fa::queries_per_workgroup(dtype == FA_DTYPE_FP32 ? fa::kDtypeFp32 : fa::kDtypeBf16);
  if (bh * ((Nq + qpw - 1) / qpw) > INT32_MAX) return FA_ERR_UNSUPPORTED;
  // one head's key rows, from its first element to the end of its last row, are addressed with 32-bit
  // offsets from a per-head buffer descriptor
  const int64_t row_stride_bytes = (layout == FA_LAYOUT_BHSD ? D : H * D) * esize;
  if ((Nk - 1) * row_stride_bytes + D * esize > INT32_MAX) return FA_ERR_UNSUPPORTED;
  if (!isfinite(scale) || !isfinite(fabsf(scale) * 1.4426950408889634f)) return FA_ERR_BAD_SCALE;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)lse) & 15) return FA_ERR_MISALIGNED;
  if (overlaps(o, bytes_q, q, bytes_q) || overlaps(o, bytes_q, k, bytes_k) || overlaps(o, bytes_q, v, bytes_k) ||
      overlaps(lse, lse_bytes, q, bytes_q) || overlaps(lse, lse_bytes, k, bytes_k) ||
      overlaps(lse, lse_bytes, v, bytes_k) || overlaps(lse, lse_bytes, o, bytes_q))
    return FA_ERR_ALIAS;

  // ---- device residency ----
  int device = 0;
  hipError_t e = hipGetDevice(&device);
  if (e != hipSuccess) {
    set_error("hipGetDevice", e);
    return FA_ERR_HIP;
  }
  const void* ptrs[5] = {q, k, v, o, lse};
  for (const void* ptr : ptrs) {
    const int st = check_device(ptr, device);
    if (st != FA_OK) return st;
  }

  // ---- launch ----
  fa::Params p;
  memset(&p, 0, sizeof p);
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.B = (int)B;
  p.H = (int)H;
  p.Nq = (int)Nq;
  p.Nkv = (int)kv_len;
  p.kv_start = kv_start;
  p.delta = q_offset - kv_start;
  // a window reaching before every key the queries could see hides nothing
  p.window = (window < 0 || window >= q_offset + Nq) ? -1 : window;
  if (layout == FA_LAYOUT_BHSD) {
    p.stride_b_q = H * Nq * D;
    p.stride_h_q = Nq * D;
    p.stride_b_k = H * Nk * D;
    p.stride_h_k = Nk * D;
    p.stride_s = D;
  } else {
    p.stride_b_q = Nq * H * D;
    p.stride_h_q = D;
    p.stride_b_k = Nk * H * D;
    p.stride_h_k = D;
    p.stride_s = H * D;
  }
  // |scale| * log2(e).  The kernels need it positive (masked -inf scores then give exp2(-inf) = 0); a
  // zero scale becomes FLT_MIN, which keeps every visible weight exactly 1 in fp32 for any logit below
  // about 2^100 in magnitude, and lse = ln(count) to within FLT_MIN * |logit|.
  p.c = scale == 0.0f ? 1.17549435e-38f : fabsf(scale) * 1.4426950408889634f;
  p.qsign = scale < 0.0f ? (dtype == FA_DTYPE_FP32 ? 0x80000000u : 0x80008000u) : 0u;
  const int kd = dtype == FA_DTYPE_FP32 ? fa::kDtypeFp32 : dtype == FA_DTYPE_FP16 ? fa::kDtypeFp16 : fa::kDtypeBf16;
  e = fa::launch(p, kd, (int)D, causal != 0, (hipStream_t)stream);
  if (e != hipSuccess) {
    set_error("kernel launch", e);
    return FA_ERR_HIP;
  }
  return FA_OK;
}

FA_API int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
                  int64_t N, int64_t D, int layout, int causal, float scale, int dtype, void* stream) {
  // N bounds the key range too, so a bad N reports as a dimension or size error, never as a range error
  if (N < 1) return (!q || !k || !v || !o || !lse) ? FA_ERR_NULL
                    : (layout != FA_LAYOUT_BHSD && layout != FA_LAYOUT_BSND) ? FA_ERR_BAD_LAYOUT
                    : (dtype != FA_DTYPE_FP32 && dtype != FA_DTYPE_FP16 && dtype != FA_DTYPE_BF16) ? FA_ERR_BAD_DTYPE
                    : FA_ERR_BAD_DIM;
  return fa_fwd_ex(q, k, v, o, lse, B, H, N, N, D, layout, causal, -1, 0, 0, N, scale, dtype, stream);
}

FA_API int fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse, const int32_t* cu_seqlens_q,
                         const int32_t* cu_seqlens_k, int64_t B, int64_t H, int64_t total_q, int64_t total_k,
                         int64_t max_seqlen_q, int64_t D, int causal, float scale, int dtype, void* stream) {
  // ---- pure argument checks (no HIP calls) ----
  if (!q || !k || !v || !o || !lse || !cu_seqlens_q || !cu_seqlens_k) return FA_ERR_NULL;
  if (dtype != FA_DTYPE_FP32 && dtype != FA_DTYPE_FP16 && dtype != FA_DTYPE_BF16) return FA_ERR_BAD_DTYPE;
  if (B < 1 || H < 1 || total_q < 1 || total_k < 1 || max_seqlen_q < 1 || D < 1) return FA_ERR_BAD_DIM;
  if (D != 64 && D != 128) return FA_ERR_UNSUPPORTED;
  if (dtype == FA_DTYPE_FP32) return FA_ERR_UNSUPPORTED;
  int64_t rows_q, rows_k, elems_q, elems_k, bytes_q, bytes_k, lse_bytes, bh, cu_bytes;
  if (total_q > kMaxRows || total_k > kMaxRows || B > kMaxRows || !mul_ok(total_q, H, &rows_q) ||
      !mul_ok(total_k, H, &rows_k) || !mul_ok(rows_q, D, &elems_q) || !mul_ok(rows_k, D, &elems_k) ||
      !mul_ok(elems_q, 2, &bytes_q) || !mul_ok(elems_k, 2, &bytes_k) || !mul_ok(rows_q, 4, &lse_bytes) ||
      !mul_ok(B, H, &bh) || bh > INT32_MAX || !mul_ok(B + 1, 4, &cu_bytes))
    return FA_ERR_UNSUPPORTED;
  if (max_seqlen_q > total_q) return FA_ERR_BAD_RANGE;
  const int64_t qpw = fa::queries_per_workgroup(fa::kDtypeBf16);
  if ((bh + 7) / 8 * 8 * ((max_seqlen_q + qpw - 1) / qpw) > INT32_MAX) return FA_ERR_UNSUPPORTED;
  // every sequence's key rows lie inside [0, total_k): its per-head byte range fits a buffer descriptor
  if ((total_k - 1) * H * D * 2 + D * 2 > INT32_MAX) return FA_ERR_UNSUPPORTED;
  if (!isfinite(scale) || !isfinite(fabsf(scale) * 1.4426950408889634f)) return FA_ERR_BAD_SCALE;
  if ((((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)lse) & 15) ||
      (((uintptr_t)cu_seqlens_q | (uintptr_t)cu_seqlens_k) & 3))
    return FA_ERR_MISALIGNED;
  const void* ins[5] = {q, k, v, cu_seqlens_q, cu_seqlens_k};
  const int64_t in_bytes[5] = {bytes_q, bytes_k, bytes_k, cu_bytes, cu_bytes};
  for (int i = 0; i < 5; ++i)
    if (overlaps(o, bytes_q, ins[i], in_bytes[i]) || overlaps(lse, lse_bytes, ins[i], in_bytes[i])) return FA_ERR_ALIAS;
  if (overlaps(lse, lse_bytes, o, bytes_q)) return FA_ERR_ALIAS;

  // ---- device residency ----
  int device = 0;
  hipError_t e = hipGetDevice(&device);
  if (e != hipSuccess) {
    set_error("hipGetDevice", e);
    return FA_ERR_HIP;
  }
  const void* ptrs[7] = {q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k};
  for (const void* ptr : ptrs) {
    const int st = check_device(ptr, device);
    if (st != FA_OK) return st;
  }

  // ---- launch ----
  fa::Params p;
  memset(&p, 0, sizeof p);
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.B = (int)B;
  p.H = (int)H;
  p.Nq = (int)max_seqlen_q;
  p.window = -1;
  p.stride_h_q = D;
  p.stride_h_k = D;
  p.stride_s = H * D;
  p.cu_q = cu_seqlens_q;
  p.cu_k = cu_seqlens_k;
  p.total_q = total_q;
  p.total_k = total_k;
  p.c = scale == 0.0f ? 1.17549435e-38f : fabsf(scale) * 1.4426950408889634f;
  p.qsign = scale < 0.0f ? 0x80008000u : 0u;
  e = fa::launch_varlen(p, dtype == FA_DTYPE_FP16 ? fa::kDtypeFp16 : fa::kDtypeBf16, (int)D, causal != 0,
                        (hipStream_t)stream);
  if (e != hipSuccess) {
    set_error("kernel launch", e);
    return FA_ERR_HIP;
  }
  return FA_OK;
}

FA_API int fa_merge(const void* o_parts, const float* lse_parts, int64_t n_parts, void* o, float* lse, int64_t B,
                    int64_t H, int64_t N, int64_t D, int layout, int dtype, void* stream) {
  if (!o_parts || !lse_parts || !o || !lse) return FA_ERR_NULL;
  if (layout != FA_LAYOUT_BHSD && layout != FA_LAYOUT_BSND) return FA_ERR_BAD_LAYOUT;
  if (dtype != FA_DTYPE_FP32 && dtype != FA_DTYPE_FP16 && dtype != FA_DTYPE_BF16) return FA_ERR_BAD_DTYPE;
  if (B < 1 || H < 1 || N < 1 || D < 1 || n_parts < 1) return FA_ERR_BAD_DIM;
  if (D != 64 && D != 128) return FA_ERR_UNSUPPORTED;
  const int64_t esize = dtype == FA_DTYPE_FP32 ? 4 : 2;
  int64_t bh, rows, elems, bytes, lse_bytes, all_bytes, all_lse_bytes, threads;
  if (n_parts > INT32_MAX || !mul_ok(B, H, &bh) || !mul_ok(bh, N, &rows) || !mul_ok(rows, D, &elems) ||
      !mul_ok(elems, esize, &bytes) || !mul_ok(rows, 4, &lse_bytes) || !mul_ok(bytes, n_parts, &all_bytes) ||
      !mul_ok(lse_bytes, n_parts, &all_lse_bytes) || !mul_ok(rows, D / 8, &threads) ||
      (threads + 255) / 256 > INT32_MAX)
    return FA_ERR_UNSUPPORTED;
  if (((uintptr_t)o_parts | (uintptr_t)lse_parts | (uintptr_t)o | (uintptr_t)lse) & 15) return FA_ERR_MISALIGNED;
  if (overlaps(o, bytes, o_parts, all_bytes) || overlaps(o, bytes, lse_parts, all_lse_bytes) ||
      overlaps(lse, lse_bytes, o_parts, all_bytes) || overlaps(lse, lse_bytes, lse_parts, all_lse_bytes) ||
      overlaps(lse, lse_bytes, o, bytes))
    return FA_ERR_ALIAS;
  int device = 0;
  hipError_t e = hipGetDevice(&device);
  if (e != hipSuccess) {
    set_error("hipGetDevice", e);
    return FA_ERR_HIP;
  }
  const void* ptrs[4] = {o_parts, lse_parts, o, lse};
  for (const void* ptr : ptrs) {
    const int st = check_device(ptr, device);
    if (st != FA_OK) return st;
  }
  const int kd = dtype == FA_DTYPE_FP32 ? fa::kDtypeFp32 : dtype == FA_DTYPE_FP16 ? fa::kDtypeFp16 : fa::kDtypeBf16;
  e = fa::launch_merge(o_parts, lse_parts, (int)n_parts, o, lse, rows, B, H, N, (int)D,
                       layout == FA_LAYOUT_BSND ? 1 : 0, kd, (hipStream_t)stream);
  if (e != hipSuccess) {
    set_error("kernel launch", e);
    return FA_ERR_HIP;
  }
  return FA_OK;
}

namespace {

// fa_bwd_ex; with delta == nullptr the D workspace is the library's own per-device scratch array
// (fa_bwd_noalloc), whose size limit is checked with the other sizes and which is neither an input nor a
// caller buffer (no aliasing or residency check).
// With dq_acc != nullptr the dQ sums go to that fp32 workspace through atomic adds (fa_bwd_atomic).
int bwd_ex(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout, void* dq,
           void* dk, void* dv, float* delta, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t D, int layout,
           int causal, int64_t window, int64_t q_offset, int64_t kv_start, int64_t kv_len, float scale, int dtype,
           void* stream, float* dq_acc = nullptr) {
  const bool scratch = delta == nullptr;
  const bool atomic = dq_acc != nullptr;
  // ---- pure argument checks (no HIP calls) ----
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return FA_ERR_NULL;
  if (layout != FA_LAYOUT_BHSD && layout != FA_LAYOUT_BSND) return FA_ERR_BAD_LAYOUT;
  if (dtype != FA_DTYPE_FP32 && dtype != FA_DTYPE_FP16 && dtype != FA_DTYPE_BF16) return FA_ERR_BAD_DTYPE;
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || D < 1) return FA_ERR_BAD_DIM;
  if (D != 64 && D != 128) return FA_ERR_UNSUPPORTED;
  const int64_t esize = dtype == FA_DTYPE_FP32 ? 4 : 2;
  int64_t bh, rows_q, rows_k, elems_q, elems_k, bytes_q, bytes_k, row_bytes;
  if (Nq > kMaxRows || Nk > kMaxRows || !mul_ok(B, H, &bh) || bh > INT32_MAX || !mul_ok(bh, Nq, &rows_q) ||
      !mul_ok(bh, Nk, &rows_k) || !mul_ok(rows_q, D, &elems_q) || !mul_ok(rows_k, D, &elems_k) ||
      !mul_ok(elems_q, esize, &bytes_q) || !mul_ok(elems_k, esize, &bytes_k) || !mul_ok(rows_q, 4, &row_bytes))
    return FA_ERR_UNSUPPORTED;
  if (kv_start < 0 || kv_len < 0 || kv_start > Nk || kv_len > Nk - kv_start) return FA_ERR_BAD_RANGE;
  if (window >= 0 && !causal) return FA_ERR_BAD_RANGE;
  if (q_offset < -kMaxRows || q_offset > kMaxRows) return FA_ERR_BAD_RANGE;
  const int64_t rpw = fa::bwd_rows_per_workgroup();
  if (bh * ((Nq + rpw - 1) / rpw) > INT32_MAX || bh * ((Nk + rpw - 1) / rpw) > INT32_MAX) return FA_ERR_UNSUPPORTED;
  // one head's rows of Q/dO and of K/V are addressed with 32-bit offsets from per-head buffer descriptors
  const int64_t stride_bytes = (layout == FA_LAYOUT_BHSD ? D : H * D) * esize;
  if ((Nq - 1) * stride_bytes + D * esize > INT32_MAX || (Nk - 1) * stride_bytes + D * esize > INT32_MAX)
    return FA_ERR_UNSUPPORTED;
  if (scratch && rows_q > kNoAllocMaxRows) return FA_ERR_SCRATCH_LIMIT;
  if (atomic && dtype == FA_DTYPE_FP32) return FA_ERR_UNSUPPORTED;
  int64_t acc_bytes = 0;
  if (atomic && !mul_ok(elems_q, 4, &acc_bytes)) return FA_ERR_UNSUPPORTED;
  if (!isfinite(scale) || !isfinite(fabsf(scale) * 1.4426950408889634f)) return FA_ERR_BAD_SCALE;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)lse | (uintptr_t)dout |
       (uintptr_t)dq | (uintptr_t)dk | (uintptr_t)dv | (uintptr_t)delta | (uintptr_t)dq_acc) & 15)
    return FA_ERR_MISALIGNED;
  const void* ins[6] = {q, k, v, o, lse, dout};
  const int64_t in_bytes[6] = {bytes_q, bytes_k, bytes_k, bytes_q, row_bytes, bytes_q};
  // the caller's outputs and workspaces (the library's scratch array is none of them)
  const void* outs[5] = {dq, dk, dv};
  int64_t out_bytes[5] = {bytes_q, bytes_k, bytes_k};
  int n_outs = 3;
  if (!scratch) {
    outs[n_outs] = delta;
    out_bytes[n_outs++] = row_bytes;
  }
  if (atomic) {
    outs[n_outs] = dq_acc;
    out_bytes[n_outs++] = acc_bytes;
  }
  for (int a = 0; a < n_outs; ++a) {
    for (int i = 0; i < 6; ++i)
      if (overlaps(outs[a], out_bytes[a], ins[i], in_bytes[i])) return FA_ERR_ALIAS;
    for (int c = a + 1; c < n_outs; ++c)
      if (overlaps(outs[a], out_bytes[a], outs[c], out_bytes[c])) return FA_ERR_ALIAS;
  }

  // ---- device residency ----
  int device = 0;
  hipError_t e = hipGetDevice(&device);
  if (e != hipSuccess) {
    set_error("hipGetDevice", e);
    return FA_ERR_HIP;
  }
  for (const void* ptr : ins) {
    const int st = check_device(ptr, device);
    if (st != FA_OK) return st;
  }
  for (int a = 0; a < n_outs; ++a) {
    const int st = check_device(outs[a], device);
    if (st != FA_OK) return st;
  }
  if (scratch) {
    const int st = scratch_of_device(device, &delta);
    if (st != FA_OK) return st;
  }

  // ---- launch ----
  fa::BwdParams p;
  memset(&p, 0, sizeof p);
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.dout = dout;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.delta = delta;
  p.dq_acc = dq_acc;
  p.B = (int)B;
  p.H = (int)H;
  p.Nq = (int)Nq;
  p.Nk = (int)Nk;
  p.q_offset = q_offset;
  // a window reaching before every key the queries could see hides nothing
  p.window = (window < 0 || window >= q_offset + Nq) ? -1 : window;
  p.kv_start = (int)kv_start;
  p.kv_len = (int)kv_len;
  if (layout == FA_LAYOUT_BHSD) {
    p.stride_b_q = H * Nq * D;
    p.stride_h_q = Nq * D;
    p.stride_b_k = H * Nk * D;
    p.stride_h_k = Nk * D;
    p.stride_s = D;
  } else {
    p.stride_b_q = Nq * H * D;
    p.stride_h_q = D;
    p.stride_b_k = Nk * H * D;
    p.stride_h_k = D;
    p.stride_s = H * D;
  }
  p.c = scale * 1.4426950408889634f;
  p.scale = scale;
  const int kd = dtype == FA_DTYPE_FP32 ? fa::kDtypeFp32 : dtype == FA_DTYPE_FP16 ? fa::kDtypeFp16 : fa::kDtypeBf16;
  e = atomic ? fa::launch_bwd_atomic(p, kd, (int)D, causal != 0, (hipStream_t)stream)
             : fa::launch_bwd(p, kd, (int)D, causal != 0, (hipStream_t)stream);
  if (e != hipSuccess) {
    set_error("kernel launch", e);
    return FA_ERR_HIP;
  }
  return FA_OK;
}

}  // namespace

FA_API int fa_bwd_ex(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                     void* dq, void* dk, void* dv, float* delta, int64_t B, int64_t H, int64_t Nq, int64_t Nk,
                     int64_t D, int layout, int causal, int64_t window, int64_t q_offset, int64_t kv_start,
                     int64_t kv_len, float scale, int dtype, void* stream) {
  if (!delta) return FA_ERR_NULL;
  return bwd_ex(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, Nq, Nk, D, layout, causal, window, q_offset, kv_start,
                kv_len, scale, dtype, stream);
}

FA_API int fa_bwd_atomic(const void* q, const void* k, const void* v, const void* o, const float* lse,
                         const void* dout, void* dq, void* dk, void* dv, float* delta, float* dq_accum, int64_t B,
                         int64_t H, int64_t N, int64_t D, int layout, int causal, float scale, int dtype,
                         void* stream) {
  if (!delta || !dq_accum) return FA_ERR_NULL;
  return bwd_ex(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, N, N, D, layout, causal, -1, 0, 0, N, scale, dtype,
                stream, dq_accum);
}

FA_API int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                          const void* dout, void* dq, void* dk, void* dv, int64_t B, int64_t H, int64_t N, int64_t D,
                          int layout, int causal, float scale, int dtype, void* stream) {
  return bwd_ex(q, k, v, o, lse, dout, dq, dk, dv, nullptr, B, H, N, N, D, layout, causal, -1, 0, 0, N, scale, dtype,
                stream);
}

FA_API int fa_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const float* lse,
                         const void* dout, void* dq, void* dk, void* dv, float* delta, const int32_t* cu_seqlens_q,
                         const int32_t* cu_seqlens_k, int64_t B, int64_t H, int64_t total_q, int64_t total_k,
                         int64_t max_seqlen_q, int64_t max_seqlen_k, int64_t D, int causal, float scale, int dtype,
                         void* stream) {
  // ---- pure argument checks (no HIP calls) ----
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !delta || !cu_seqlens_q || !cu_seqlens_k)
    return FA_ERR_NULL;
  if (dtype != FA_DTYPE_FP32 && dtype != FA_DTYPE_FP16 && dtype != FA_DTYPE_BF16) return FA_ERR_BAD_DTYPE;
  if (B < 1 || H < 1 || total_q < 1 || total_k < 1 || max_seqlen_q < 1 || max_seqlen_k < 1 || D < 1)
    return FA_ERR_BAD_DIM;
  if (D != 64 && D != 128) return FA_ERR_UNSUPPORTED;
  if (dtype == FA_DTYPE_FP32) return FA_ERR_UNSUPPORTED;
  int64_t rows_q, rows_k, elems_q, elems_k, bytes_q, bytes_k, row_bytes, bh, cu_bytes;
  if (total_q > kMaxRows || total_k > kMaxRows || B > kMaxRows || !mul_ok(total_q, H, &rows_q) ||
      !mul_ok(total_k, H, &rows_k) || !mul_ok(rows_q, D, &elems_q) || !mul_ok(rows_k, D, &elems_k) ||
      !mul_ok(elems_q, 2, &bytes_q) || !mul_ok(elems_k, 2, &bytes_k) || !mul_ok(rows_q, 4, &row_bytes) ||
      !mul_ok(B, H, &bh) || bh > INT32_MAX || !mul_ok(B + 1, 4, &cu_bytes))
    return FA_ERR_UNSUPPORTED;
  if (max_seqlen_q > total_q || max_seqlen_k > total_k) return FA_ERR_BAD_RANGE;
  const int64_t rpw = fa::bwd_rows_per_workgroup();
  if ((bh + 7) / 8 * 8 * ((max_seqlen_q + rpw - 1) / rpw) > INT32_MAX ||
      (bh + 7) / 8 * 8 * ((max_seqlen_k + rpw - 1) / rpw) > INT32_MAX)
    return FA_ERR_UNSUPPORTED;
  // every sequence's rows lie inside [0, total): one head's rows fit a buffer descriptor
  if ((total_q - 1) * H * D * 2 + D * 2 > INT32_MAX || (total_k - 1) * H * D * 2 + D * 2 > INT32_MAX)
    return FA_ERR_UNSUPPORTED;
  if (!isfinite(scale) || !isfinite(fabsf(scale) * 1.4426950408889634f)) return FA_ERR_BAD_SCALE;
  if ((((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)lse | (uintptr_t)dout |
        (uintptr_t)dq | (uintptr_t)dk | (uintptr_t)dv | (uintptr_t)delta) & 15) ||
      (((uintptr_t)cu_seqlens_q | (uintptr_t)cu_seqlens_k) & 3))
    return FA_ERR_MISALIGNED;
  const void* ins[8] = {q, k, v, o, lse, dout, cu_seqlens_q, cu_seqlens_k};
  const int64_t in_bytes[8] = {bytes_q, bytes_k, bytes_k, bytes_q, row_bytes, bytes_q, cu_bytes, cu_bytes};
  const void* outs[4] = {dq, dk, dv, delta};
  const int64_t out_bytes[4] = {bytes_q, bytes_k, bytes_k, row_bytes};
  for (int a = 0; a < 4; ++a) {
    for (int i = 0; i < 8; ++i)
      if (overlaps(outs[a], out_bytes[a], ins[i], in_bytes[i])) return FA_ERR_ALIAS;
    for (int c = a + 1; c < 4; ++c)
      if (overlaps(outs[a], out_bytes[a], outs[c], out_bytes[c])) return FA_ERR_ALIAS;
  }

  // ---- device residency ----
  int device = 0;
  hipError_t e = hipGetDevice(&device);
  if (e != hipSuccess) {
    set_error("hipGetDevice", e);
    return FA_ERR_HIP;
  }
  for (const void* ptr : ins) {
    const int st = check_device(ptr, device);
    if (st != FA_OK) return st;
  }
  for (const void* ptr : outs) {
    const int st = check_device(ptr, device);
    if (st != FA_OK) return st;
  }

  // ---- launch ----
  fa::BwdParams p;
  memset(&p, 0, sizeof p);
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.dout = dout;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.delta = delta;
  p.B = (int)B;
  p.H = (int)H;
  p.Nq = (int)max_seqlen_q;
  p.Nk = (int)max_seqlen_k;
  p.window = -1;
  p.stride_h_q = D;
  p.stride_h_k = D;
  p.stride_s = H * D;
  p.cu_q = cu_seqlens_q;
  p.cu_k = cu_seqlens_k;
  p.total_q = total_q;
  p.total_k = total_k;
  p.c = scale * 1.4426950408889634f;
  p.scale = scale;
  e = fa::launch_bwd_varlen(p, dtype == FA_DTYPE_FP16 ? fa::kDtypeFp16 : fa::kDtypeBf16, (int)D, causal != 0,
                            (hipStream_t)stream);
  if (e != hipSuccess) {
    set_error("kernel launch", e);
    return FA_ERR_HIP;
  }
  return FA_OK;
}

FA_API int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                  void* dq, void* dk, void* dv, float* delta, int64_t B, int64_t H, int64_t N, int64_t D,
                  int layout, int causal, float scale, int dtype, void* stream) {
  // the whole key range: a bad N is reported by the dimension and size checks, which come first
  return fa_bwd_ex(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, N, N, D, layout, causal, -1, 0, 0, N, scale,
                   dtype, stream);
}
