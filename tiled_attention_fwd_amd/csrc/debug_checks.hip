// Device-resident precondition checks, run only when ATTN_FWD_DEBUG is set.
//
// The host cannot see cu_seqlens, indices or seqlens_k without a copy, so the
// ABI documents them as preconditions.  In debug mode the library launches
// these small kernels before the real work, reads back one status word and
// returns ATTN_ERR_SHAPE instead of launching on inconsistent metadata.  The
// checks only read the arrays within the sizes the caller declares.

#include "attn_internal.h"

namespace attnfwd {
namespace {

// Status bits (OR-ed by the checks; 0 = consistent).
constexpr int kCuFirst = 1, kCuOrder = 2, kCuLast = 4, kCuTooLong = 8, kIdxRange = 16,
              kIdxOrder = 32, kIdxRuns = 64;

__device__ int g_status;

__global__ __launch_bounds__(256) void reset_status_kernel() {
  if (threadIdx.x == 0) g_status = 0;
}

// cu (n + 1 entries): cu[0] == 0, nondecreasing, cu[n] == total, every
// difference <= max_len (max_len < 0: not checked).
__global__ __launch_bounds__(256) void check_cu_kernel(const int32_t* cu, int n, int total,
                                                       int max_len) {
  int bad = 0;
  for (int i = threadIdx.x; i < n; i += 256) {
    const int a = cu[i], b = cu[i + 1];
    if (b < a) bad |= kCuOrder;
    if (max_len >= 0 && b - a > max_len) bad |= kCuTooLong;
  }
  if (threadIdx.x == 0) {
    if (cu[0] != 0) bad |= kCuFirst;
    if (cu[n] != total) bad |= kCuLast;
  }
  if (bad) atomicOr(&g_status, bad);
}

// lens (n entries): 0 <= lens[i] <= max_len.
__global__ __launch_bounds__(256) void check_lens_kernel(const int32_t* lens, int n, int max_len) {
  int bad = 0;
  for (int i = threadIdx.x; i < n; i += 256)
    if (lens[i] < 0 || lens[i] > max_len) bad |= kCuTooLong;
  if (bad) atomicOr(&g_status, bad);
}

// idx (n entries): strictly increasing, and 0 <= idx[i] < n_rows unless
// n_rows < 0.
__global__ __launch_bounds__(256) void check_indices_kernel(const int32_t* idx, int n, int n_rows) {
  int bad = 0;
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) {
    const int v = idx[i];
    if (n_rows >= 0 && (v < 0 || v >= n_rows)) bad |= kIdxRange;
    if (i > 0 && idx[i - 1] >= v) bad |= kIdxOrder;
  }
  if (bad) atomicOr(&g_status, bad);
}

// The rows of each sequence are consecutive in the padded tensor: for every
// i in (cu[s], cu[s+1]), idx[i] == idx[i-1] + 1.  The sequence of entry i is
// found by binary search over cu (n + 1 entries, n >= 1); the search stays
// within cu whatever its contents, and only idx[0..n_idx) is read.
__global__ __launch_bounds__(256) void check_runs_kernel(const int32_t* idx, int n_idx,
                                                         const int32_t* cu, int n) {
  int bad = 0;
  for (int i = blockIdx.x * 256 + threadIdx.x + 1; i < n_idx; i += gridDim.x * 256) {
    int lo = 0, hi = n - 1;  // the last sequence whose start is <= i
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (cu[mid] <= i) lo = mid;
      else hi = mid - 1;
    }
    if (cu[lo] < i && idx[i] != idx[i - 1] + 1) bad |= kIdxRuns;
  }
  if (bad) atomicOr(&g_status, bad);
}

}  // namespace

hipError_t debug_reset(hipStream_t s) {
  hipLaunchKernelGGL(reset_status_kernel, dim3(1), dim3(256), 0, s);
  return hipGetLastError();
}

hipError_t debug_check_cu(const int32_t* cu, int n, int total, int max_len, hipStream_t s) {
  if (n < 0) return hipSuccess;
  hipLaunchKernelGGL(check_cu_kernel, dim3(1), dim3(256), 0, s, cu, n, total, max_len);
  return hipGetLastError();
}

hipError_t debug_check_lens(const int32_t* lens, int n, int max_len, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(check_lens_kernel, dim3(1), dim3(256), 0, s, lens, n, max_len);
  return hipGetLastError();
}

hipError_t debug_check_indices(const int32_t* idx, int n, int n_rows, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int blocks = (n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024;
  hipLaunchKernelGGL(check_indices_kernel, dim3(blocks), dim3(256), 0, s, idx, n, n_rows);
  return hipGetLastError();
}

hipError_t debug_check_runs(const int32_t* idx, int n_idx, const int32_t* cu, int n,
                            hipStream_t s) {
  if (n_idx <= 1 || n <= 0) return hipSuccess;
  const int blocks = (n_idx + 255) / 256 < 1024 ? (n_idx + 255) / 256 : 1024;
  hipLaunchKernelGGL(check_runs_kernel, dim3(blocks), dim3(256), 0, s, idx, n_idx, cu, n);
  return hipGetLastError();
}

// Waits for the stream and returns the status word (-1 if HIP failed).
int debug_status(hipStream_t s) {
  if (hipStreamSynchronize(s) != hipSuccess) return -1;
  int v = 0;
  if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_status), sizeof(int), 0, hipMemcpyDeviceToHost) !=
      hipSuccess)
    return -1;
  return v;
}

}  // namespace attnfwd
