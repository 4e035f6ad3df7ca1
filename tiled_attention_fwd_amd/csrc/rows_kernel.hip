// Row gather (unpad) and row scatter (pad) for the packed attention path.
//
// Page "Lesson 5: IAW model FA2 vs FA3 measured", section 1: the padded
// (B, total_len, H, D) tensor is compacted by gathering the rows named by
// `indices`, attention runs on the compact rows, and the result is scattered
// back to the padded positions.  Sections 2 and 6 show these moves as one
// gather per tensor and a fill kernel followed by an index-put kernel.  Here
// one launch gathers q, k and v together, and one launch writes every padded
// output row exactly once (copied row or zeros), so no separate fill runs.
//
// Both kernels are pure HBM streams: 16-byte vector loads and stores, each
// lane moving consecutive 16-byte chunks of a row so a wave covers 1 KiB of
// contiguous bytes per instruction.

#include "attn_internal.h"

namespace attnfwd {
namespace {

constexpr int kThreads = 256;

// The padded output of the scatter is written once and read by nothing that
// follows on the path: streaming (nontemporal) stores keep it from displacing
// useful lines.  (The gather's output is read right away by the attention, so
// it stays on normal stores: streaming it measured slower end to end.)
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store_stream(uint4* p, uint4 v) {
  __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v), reinterpret_cast<u32x4*>(p));
}
constexpr int kUnroll = 4;  // 16-byte chunks per thread per pass

struct GatherArgs {
  const uint4* src[3];
  uint4* dst[3];
  const int32_t* indices;
  int32_t n_valid;
  int32_t n_rows_src;
  int32_t cpr;      // 16-byte chunks per row
  int64_t total;    // n_valid * cpr chunks per tensor
};

__global__ __launch_bounds__(kThreads) void gather_rows_kernel(const GatherArgs a) {
  const int t = blockIdx.y;
  const uint4* __restrict__ src = a.src[t];
  uint4* __restrict__ dst = a.dst[t];
  const int64_t base = (int64_t)blockIdx.x * kThreads * kUnroll + threadIdx.x;
  uint4 val[kUnroll];
  int64_t out_at[kUnroll];
#pragma unroll
  for (int i = 0; i < kUnroll; ++i) {
    const int64_t g = base + (int64_t)i * kThreads;
    out_at[i] = -1;
    if (g < a.total) {
      // total < 2^32 is checked on the host, so 32-bit division is exact here
      const uint32_t row = (uint32_t)g / (uint32_t)a.cpr;
      const uint32_t col = (uint32_t)g - row * (uint32_t)a.cpr;
      const int idx = a.indices[row];
      val[i] = (idx >= 0 && idx < a.n_rows_src) ? src[(int64_t)idx * a.cpr + col]
                                                : make_uint4(0, 0, 0, 0);
      out_at[i] = g;
    }
  }
#pragma unroll
  for (int i = 0; i < kUnroll; ++i)
    if (out_at[i] >= 0) dst[out_at[i]] = val[i];  // read next by the attention: keep cached
}

// Scatter: each workgroup owns kRows consecutive destination rows.  Because
// `indices` is strictly increasing, the source rows that land in
// [r0, r0 + kRows) are the (at most kRows) entries starting at the first
// position whose index is >= r0.  Wave 0 finds that position with a 64-way
// search (each round probes 64 evenly spaced entries, so 65536 entries take
// three dependent rounds), then the workgroup builds a row -> source map in
// LDS and streams the rows.
constexpr int kRows = 8;

__device__ int lower_bound_wave(const int32_t* idx, int n, int key, int lane) {
  int lo = 0, hi = n;  // answer in [lo, hi]
  while (hi - lo > 0) {
    const int span = hi - lo;
    const int step = (span + 63) / 64;
    const int pos = lo + lane * step;
    const bool probe = pos < hi;
    const bool less = probe && idx[pos] < key;
    const uint64_t m = __ballot(less);
    const int cnt = __popcll(m);
    // Probes 0..cnt-1 are < key, so the answer is in (lo + (cnt-1)*step, lo + cnt*step].
    const int new_lo = cnt > 0 ? lo + (cnt - 1) * step + 1 : lo;
    const int new_hi = min(hi, lo + cnt * step);
    if (step == 1) return min(hi, lo + cnt);
    lo = new_lo;
    hi = new_hi;
  }
  return lo;
}

__global__ __launch_bounds__(kThreads) void scatter_rows_kernel(
    const uint4* __restrict__ src, uint4* __restrict__ dst, const int32_t* __restrict__ indices,
    int n_valid, int n_rows_total, int cpr) {
  __shared__ int pos0_s;
  __shared__ int srcpos[kRows];
  const int r0 = blockIdx.x * kRows;
  const int tid = threadIdx.x;
  if (tid < 64) {
    const int p0 = lower_bound_wave(indices, n_valid, r0, tid);
    if (tid == 0) pos0_s = p0;
  }
  if (tid < kRows) srcpos[tid] = -1;
  __syncthreads();
  if (tid < kRows) {
    const int p = pos0_s + tid;
    if (p < n_valid) {
      const int r = indices[p];
      if (r >= r0 && r < r0 + kRows && r < n_rows_total) srcpos[r - r0] = p;
    }
  }
  __syncthreads();
  const int nrows = min(kRows, n_rows_total - r0);
  const int total = nrows * cpr;
  // batches of kScatterBatch chunks per thread: every load of a batch is
  // issued before its stores, so each thread keeps several rows in flight
  constexpr int kScatterBatch = 8;
  for (int g0 = 0; g0 < total; g0 += kThreads * kScatterBatch) {
    uint4 v[kScatterBatch];
    int64_t at[kScatterBatch];
#pragma unroll
    for (int i = 0; i < kScatterBatch; ++i) {
      const int g = g0 + i * kThreads + tid;
      at[i] = -1;
      v[i] = make_uint4(0, 0, 0, 0);
      if (g < total) {
        const int row = g / cpr;
        const int col = g - row * cpr;
        const int sp = srcpos[row];
        if (sp >= 0 && src == nullptr) continue;  // fill only: indexed rows stay as they are
        if (sp >= 0) v[i] = src[(int64_t)sp * cpr + col];
        at[i] = (int64_t)(r0 + row) * cpr + col;
      }
    }
#pragma unroll
    for (int i = 0; i < kScatterBatch; ++i)
      if (at[i] >= 0) store_stream(&dst[at[i]], v[i]);
  }
}

// ---- padding mask -> (indices, cu_seqlens, n_valid, max_seqlen)
//
// Page "Lesson 5: IAW model FA2 vs FA3 measured", section 1: unpad gathers
// the non-padding rows named by `indices`, and the varlen attention needs the
// sequence offsets.  The padded tensor is B slots of L rows; a nonzero mask
// byte marks a valid row; slot b's valid rows form sequence b.  Three small
// launches: per-slot counts, one scan, per-slot index writes in row order.

__global__ __launch_bounds__(256) void mask_count_kernel(const uint8_t* __restrict__ mask, int L,
                                                         int32_t* __restrict__ cu) {
  __shared__ int part[4];
  const uint8_t* row = mask + (int64_t)blockIdx.x * L;
  int n = 0;
  for (int i = threadIdx.x; i < L; i += 256) n += row[i] != 0;
  for (int off = 32; off > 0; off >>= 1) n += __shfl_xor(n, off);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = n;
  __syncthreads();
  if (threadIdx.x == 0) cu[blockIdx.x + 1] = part[0] + part[1] + part[2] + part[3];
}

// In-place running sums of cu[1..B] (the counts), cu[0] = 0, and
// stats = {n_valid, max count}.  One workgroup of 1024 threads.
__global__ __launch_bounds__(1024) void mask_scan_kernel(int32_t* __restrict__ cu, int B,
                                                         int32_t* __restrict__ stats) {
  __shared__ int wsum[16];
  __shared__ int wmax[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int carry = 0, mx = 0;
  for (int base = 0; base < B; base += 1024) {
    const int i = base + tid;
    const int v = i < B ? cu[i + 1] : 0;
    mx = max(mx, v);
    int x = v;
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    if (wave == 0) {
      int w = lane < 16 ? wsum[lane] : 0;
      for (int off = 1; off < 16; off <<= 1) {
        const int y = __shfl_up(w, off);
        if (lane >= off) w += y;
      }
      if (lane < 16) wsum[lane] = w;
    }
    __syncthreads();
    if (i < B) cu[i + 1] = carry + (wave > 0 ? wsum[wave - 1] : 0) + x;
    carry += wsum[15];
    __syncthreads();
  }
  for (int off = 32; off > 0; off >>= 1) mx = max(mx, __shfl_xor(mx, off));
  if (lane == 0) wmax[wave] = mx;
  __syncthreads();
  if (tid == 0) {
    int m = 0;
    for (int w = 0; w < 16; ++w) m = max(m, wmax[w]);
    cu[0] = 0;
    stats[0] = carry;
    stats[1] = m;
  }
}

__global__ __launch_bounds__(256) void mask_index_kernel(const uint8_t* __restrict__ mask, int L,
                                                         const int32_t* __restrict__ cu,
                                                         int32_t* __restrict__ indices) {
  __shared__ int wcnt[4];
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint8_t* row = mask + (int64_t)b * L;
  const int out0 = cu[b];
  int carry = 0;
  for (int c0 = 0; c0 < L; c0 += 256) {
    const int i = c0 + tid;
    const bool v = i < L && row[i] != 0;
    const uint64_t bal = __ballot(v);
    const int before = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) wcnt[wave] = __popcll(bal);
    __syncthreads();
    int pre = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int c = wcnt[w];
      pre += w < wave ? c : 0;
      tot += c;
    }
    if (v) indices[out0 + carry + pre + before] = b * L + i;
    carry += tot;
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_gather(const void* const* src, void* const* dst, int n_tensors,
                         const int32_t* indices, int n_valid, int n_rows_src, int64_t row_bytes,
                         hipStream_t stream) {
  GatherArgs a{};
  for (int t = 0; t < n_tensors; ++t) {
    a.src[t] = static_cast<const uint4*>(src[t]);
    a.dst[t] = static_cast<uint4*>(dst[t]);
  }
  a.indices = indices;
  a.n_valid = n_valid;
  a.n_rows_src = n_rows_src;
  a.cpr = (int32_t)(row_bytes / 16);
  a.total = (int64_t)n_valid * a.cpr;
  const int64_t blocks = (a.total + kThreads * kUnroll - 1) / (kThreads * kUnroll);
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(gather_rows_kernel, dim3((unsigned)blocks, n_tensors), dim3(kThreads), 0,
                     stream, a);
  return hipGetLastError();
}

hipError_t launch_scatter(const void* src, void* dst, const int32_t* indices, int n_valid,
                          int n_rows_total, int64_t row_bytes, hipStream_t stream) {
  const int cpr = (int)(row_bytes / 16);
  const int blocks = (n_rows_total + kRows - 1) / kRows;
  hipLaunchKernelGGL(scatter_rows_kernel, dim3(blocks), dim3(kThreads), 0, stream,
                     static_cast<const uint4*>(src), static_cast<uint4*>(dst), indices, n_valid,
                     n_rows_total, cpr);
  return hipGetLastError();
}

}  // namespace attnfwd

namespace attnfwd {

hipError_t launch_mask_to_varlen(const uint8_t* mask, int B, int L, int32_t* indices,
                                 int32_t* cu_seqlens, int32_t* stats, hipStream_t stream) {
  if (B > 0)  // L == 0 is fine: every count is 0
    hipLaunchKernelGGL(mask_count_kernel, dim3(B), dim3(256), 0, stream, mask, L, cu_seqlens);
  hipLaunchKernelGGL(mask_scan_kernel, dim3(1), dim3(1024), 0, stream, cu_seqlens, B, stats);
  if (B > 0)
    hipLaunchKernelGGL(mask_index_kernel, dim3(B), dim3(256), 0, stream, mask, L, cu_seqlens, indices);
  return hipGetLastError();
}

}  // namespace attnfwd
