// Microbenchmarks that ground the roofline figures used for the attention
// kernel on gfx950: MFMA bf16 32x32x16 rate, v_exp_f32 and v_fma_f32 issue
// rates, LDS read bandwidth (16-byte, 8-byte and 8-byte transposing reads), a plain 16-byte copy kernel (its known
// byte count calibrates the HBM traffic counters), and the MFMA rate with
// independent VALU, exp and LDS work mixed in at 2 waves per SIMD (the
// ceiling for the attention loop's instruction mix), and two read-only HBM
// streams (16-byte loads into registers; LDS DMA of 1 KiB per wave
// instruction with a few groups in flight) that bound the memory-bound
// kernels.
//
// Prints one JSON object.  Every kernel only touches buffers it allocates, with
// indices bounded by the launch shape.

#include <hip/hip_runtime.h>
#include <stdio.h>
#include <stdlib.h>

#include "attn_device.h"

using attnfwd::bf16x8;
using attnfwd::f32x16;

#define CHECK(x)                                                             \
  do {                                                                       \
    hipError_t e_ = (x);                                                     \
    if (e_ != hipSuccess) {                                                  \
      fprintf(stderr, "HIP error %s at %s:%d\n", hipGetErrorString(e_), __FILE__, __LINE__); \
      exit(1);                                                               \
    }                                                                        \
  } while (0)

constexpr int kIters = 2048;

__global__ __launch_bounds__(256) void mfma_kernel(float* out, float seed) {
  bf16x8 a, b;
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(seed * (threadIdx.x + e));
    b[e] = (__bf16)(seed * (e + 1));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < kIters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.f;
  for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void exp_kernel(float* out, float seed) {
  float x[8];
  for (int j = 0; j < 8; ++j) x[j] = seed * (threadIdx.x + j) * 1e-6f;
  for (int i = 0; i < kIters; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = __builtin_amdgcn_exp2f(x[j]) - 1.0f;
  }
  float s = 0.f;
  for (int j = 0; j < 8; ++j) s += x[j];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void exp_only_kernel(float* out, float seed) {
  // exp2 of exp2: no extra VALU op between transcendental instructions
  float x[8];
  for (int j = 0; j < 8; ++j) x[j] = -seed * (threadIdx.x + j);
  for (int i = 0; i < kIters; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = -__builtin_amdgcn_exp2f(x[j]);
  }
  float s = 0.f;
  for (int j = 0; j < 8; ++j) s += x[j];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void fma_kernel(float* out, float seed) {
  float x[8];
  for (int j = 0; j < 8; ++j) x[j] = seed * (threadIdx.x + j);
  for (int i = 0; i < kIters; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = fmaf(x[j], 0.999f, 0.001f);
  }
  float s = 0.f;
  for (int j = 0; j < 8; ++j) s += x[j];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void lds_kernel(float* out) {
  __shared__ __attribute__((aligned(16))) uint4 buf[4096];  // 64 KiB
  for (int i = threadIdx.x; i < 4096; i += 256) buf[i] = make_uint4(i, i + 1, i + 2, i + 3);
  __syncthreads();
  uint4 acc = make_uint4(0, 0, 0, 0);
  // independent 16-byte reads: addresses depend on the loop counter only
  for (int i = 0; i < kIters; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint4 v = buf[(threadIdx.x + j * 256 + i * 64) & 4095];
      acc.x ^= v.x; acc.y ^= v.y; acc.z ^= v.z; acc.w ^= v.w;
    }
  }
  out[blockIdx.x * blockDim.x + threadIdx.x] = (float)(acc.x ^ acc.y ^ acc.z ^ acc.w);
}

// 8-byte LDS reads, plain (ds_read_b64) or transposing (ds_read_b64_tr_b16,
// the V operand read of the attention loop): each wave reads 512 contiguous
// bytes per instruction, offsets wrap inside the 64 KiB buffer.
template <bool TR>
__global__ __launch_bounds__(256) void lds8_kernel(float* out) {
  __shared__ __attribute__((aligned(16))) uint4 buf[4096];  // 64 KiB
  for (int i = threadIdx.x; i < 4096; i += 256) buf[i] = make_uint4(i, i + 1, i + 2, i + 3);
  __syncthreads();
  const uint16_t* b16 = reinterpret_cast<const uint16_t*>(buf);
  uint2 acc = make_uint2(0, 0);
  for (int i = 0; i < kIters; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int e = (threadIdx.x * 4 + j * 1024 + i * 256) & 32767;  // element offset, 8-byte aligned
      uint2 v;
      if constexpr (TR) v = attnfwd::ds_read_tr16(b16 + e);
      else v = *reinterpret_cast<const uint2*>(b16 + e);
      acc.x ^= v.x; acc.y ^= v.y;
    }
  }
  out[blockIdx.x * blockDim.x + threadIdx.x] = (float)(acc.x ^ acc.y);
}

__global__ __launch_bounds__(256) void copy_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                  long n) {
  long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  long stride = (long)gridDim.x * blockDim.x;
  for (; i < n; i += stride) dst[i] = src[i];
}

// Read-only stream into registers: four independent 16-byte loads per thread
// in flight, XOR-folded so the loads are not dead.
__global__ __launch_bounds__(256) void read_kernel(const uint4* __restrict__ src, long n,
                                                  unsigned* __restrict__ out) {
  const long stride = (long)gridDim.x * blockDim.x;
  long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  uint4 acc = make_uint4(0, 0, 0, 0);
  for (; i + 3 * stride < n; i += 4 * stride) {
    const uint4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    acc.x ^= a.x ^ b.x ^ c.x ^ d.x;
    acc.y ^= a.y ^ b.y ^ c.y ^ d.y;
    acc.z ^= a.z ^ b.z ^ c.z ^ d.z;
    acc.w ^= a.w ^ b.w ^ c.w ^ d.w;
  }
  for (; i < n; i += stride) {
    const uint4 a = src[i];
    acc.x ^= a.x;
    acc.y ^= a.y;
    acc.z ^= a.z;
    acc.w ^= a.w;
  }
  out[(long)blockIdx.x * blockDim.x + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

// Read-only stream through LDS DMA: each wave moves groups of 4 KiB (four
// 1 KiB buffer_load ... lds instructions) into its own STAGES-deep ring and
// keeps STAGES - 1 groups in flight.  n_groups * 4096 bytes must lie inside
// the descriptor (the caller passes the buffer size).
template <int STAGES>
__global__ __launch_bounds__(256) void read_dma_kernel(const void* src, uint32_t bytes, long n_groups,
                                                      unsigned* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[4 * STAGES * 4096];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const attnfwd::u32x4 desc = attnfwd::make_desc(src, bytes);
  const uint32_t base = attnfwd::lds_addr(lds) + wave * STAGES * 4096;
  const long step = (long)gridDim.x * 4;
  int s = 0;
  for (long g = (long)blockIdx.x * 4 + wave; g < n_groups; g += step) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      attnfwd::dma16(desc, (uint32_t)(g * 4096 + j * 1024 + lane * 16),
                     __builtin_amdgcn_readfirstlane(base + s * 4096 + j * 1024));
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(4 * (STAGES - 1)) : "memory");
    s = s + 1 == STAGES ? 0 : s + 1;
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  out[(long)blockIdx.x * blockDim.x + threadIdx.x] =
      reinterpret_cast<const unsigned*>(lds)[threadIdx.x];
}

// Per MFMA: NV independent v_fma_f32, NX v_exp_f32, NL 16-byte LDS reads
// (each feeding a later MFMA's A operand), and NT pairs of transposing 8-byte
// reads (the V operand of the attention loop's P V products); with ALT the
// 16-byte reads go with even MFMAs and the transposing pairs with odd ones,
// as the score and P V halves of the attention loop alternate.  Two
// accumulators alternate.
constexpr int kMixIters = 256;
template <int NV, int NX, int NL, int NT = 0, bool ALT = false>
__global__ void mix_kernel(float* out, float seed) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  const int lane = threadIdx.x & 63;
  for (int i = threadIdx.x; i < 8192; i += blockDim.x) reinterpret_cast<float*>(lds)[i] = seed * i;
  __syncthreads();
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(seed * (threadIdx.x + i));
    b[i] = (__bf16)(seed * i);
  }
  f32x16 acc0 = {}, acc1 = {};
  float v[16];
  for (int i = 0; i < 16; ++i) v[i] = seed * (i + lane);
  for (int it = 0; it < kMixIters; ++it) {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      if (k & 1) acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc1, 0, 0, 0);
      else acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc0, 0, 0, 0);
#pragma unroll
      for (int j = 0; j < NV; ++j) v[(k * 3 + j) & 15] = fmaf(v[(k * 3 + j) & 15], seed, 0.5f);
#pragma unroll
      for (int j = 0; j < NX; ++j) v[(k * 5 + j + 7) & 15] = __builtin_amdgcn_exp2f(v[(k * 5 + j + 7) & 15]);
#pragma unroll
      for (int j = 0; j < NL; ++j) {
        if (ALT && (k & 1)) continue;
        // offsets stay below 32 KiB of the 100 KiB dynamic LDS
        const uint4 u = *reinterpret_cast<const uint4*>(lds + ((lane * 16 + (k * NL + j) * 1024 + it * 64) & 32767));
        a = __builtin_bit_cast(bf16x8, u);
      }
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        if (ALT && !(k & 1)) continue;
        const int e = (lane * 4 + (k * NT + j) * 512 + it * 32) & 16383;  // elements, below 32 KiB
        const uint16_t* b16 = reinterpret_cast<const uint16_t*>(lds);
        const uint2 lo = attnfwd::ds_read_tr16(b16 + e);
        const uint2 hi = attnfwd::ds_read_tr16(b16 + ((e + 256) & 16383));
        a = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
      }
    }
  }
  float s = 0.f;
  for (int r = 0; r < 16; ++r) s += acc0[r] + acc1[r] + v[r];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

template <typename F>
float time_ms(F launch, int reps) {
  hipEvent_t a, b;
  CHECK(hipEventCreate(&a));
  CHECK(hipEventCreate(&b));
  launch();
  CHECK(hipDeviceSynchronize());
  CHECK(hipEventRecord(a, 0));
  for (int i = 0; i < reps; ++i) launch();
  CHECK(hipEventRecord(b, 0));
  CHECK(hipEventSynchronize(b));
  float ms = 0.f;
  CHECK(hipEventElapsedTime(&ms, a, b));
  CHECK(hipEventDestroy(a));
  CHECK(hipEventDestroy(b));
  return ms / reps;
}

int main(int argc, char** argv) {
  long copy_bytes = argc > 1 ? atol(argv[1]) : (1L << 30);
  hipDeviceProp_t prop;
  CHECK(hipGetDeviceProperties(&prop, 0));
  const int cus = prop.multiProcessorCount;
  const int blocks = cus * 8;  // 8 workgroups of 4 waves per CU: 8 waves per SIMD
  float* out;
  CHECK(hipMalloc(&out, (size_t)blocks * 256 * sizeof(float)));

  const double waves = (double)blocks * 4;
  double ms;

  ms = time_ms([&] { hipLaunchKernelGGL(mfma_kernel, dim3(blocks), dim3(256), 0, 0, out, 1e-3f); }, 5);
  const double mfma_flops = waves * kIters * 4 * 32.0 * 32 * 16 * 2;
  const double mfma_tflops = mfma_flops / (ms * 1e-3) / 1e12;

  ms = time_ms([&] { hipLaunchKernelGGL(exp_kernel, dim3(blocks), dim3(256), 0, 0, out, 1.0f); }, 5);
  const double exp_sub_ops = waves * 64.0 * kIters * 8;  // lane-ops of exp (+ one sub each)
  const double exp_sub_rate = exp_sub_ops / (ms * 1e-3) / 1e12;

  ms = time_ms([&] { hipLaunchKernelGGL(exp_only_kernel, dim3(blocks), dim3(256), 0, 0, out, 1.0f); }, 5);
  const double exp_rate = exp_sub_ops / (ms * 1e-3) / 1e12;

  ms = time_ms([&] { hipLaunchKernelGGL(fma_kernel, dim3(blocks), dim3(256), 0, 0, out, 1.0f); }, 5);
  const double fma_rate = waves * 64.0 * kIters * 8 / (ms * 1e-3) / 1e12;

  ms = time_ms([&] { hipLaunchKernelGGL(lds_kernel, dim3(cus * 2), dim3(256), 0, 0, out); }, 5);
  const double lds_bytes = (double)cus * 2 * 256 * kIters * 8 * 16;
  const double lds_tbs = lds_bytes / (ms * 1e-3) / 1e12;
  ms = time_ms([&] { hipLaunchKernelGGL(lds8_kernel<false>, dim3(cus * 2), dim3(256), 0, 0, out); }, 5);
  const double lds8_tbs = lds_bytes / 2 / (ms * 1e-3) / 1e12;
  ms = time_ms([&] { hipLaunchKernelGGL(lds8_kernel<true>, dim3(cus * 2), dim3(256), 0, 0, out); }, 5);
  const double lds8tr_tbs = lds_bytes / 2 / (ms * 1e-3) / 1e12;

  // MFMA rate with mixed-in work: 512 threads and 100 KiB of LDS per workgroup,
  // one workgroup per CU = 2 waves per SIMD
  const size_t mix_lds = 100 * 1024;
  auto mix = [&](auto kern) {
    CHECK(hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, mix_lds));
    const double ms_ = time_ms([&] { hipLaunchKernelGGL(kern, dim3(cus), dim3(512), mix_lds, 0, out, 1e-3f); }, 5);
    return (double)cus * 8 * kMixIters * 16 * 32768.0 / (ms_ * 1e-3) / 1e12;
  };
  const double mix_pure = mix(mix_kernel<0, 0, 0>);
  const double mix_v4 = mix(mix_kernel<4, 0, 0>);
  const double mix_x1 = mix(mix_kernel<0, 1, 0>);
  const double mix_l1 = mix(mix_kernel<0, 0, 1>);
  const double mix_all = mix(mix_kernel<4, 1, 1>);
  const double mix_t1 = mix(mix_kernel<0, 0, 0, 1>);
  const double mix_all_t = mix(mix_kernel<4, 1, 0, 1>);
  const double mix_alt = mix(mix_kernel<4, 1, 1, 1, true>);

  uint4 *src, *dst;
  const long n = copy_bytes / 16;
  CHECK(hipMalloc(&src, n * 16));
  CHECK(hipMalloc(&dst, n * 16));
  CHECK(hipMemset(src, 1, n * 16));
  ms = time_ms([&] { hipLaunchKernelGGL(copy_kernel, dim3(cus * 16), dim3(256), 0, 0, src, dst, n); }, 10);
  const double copy_gbs = 2.0 * n * 16 / (ms * 1e-3) / 1e9;

  unsigned* rout;
  const int rblocks = cus * 8;
  CHECK(hipMalloc(&rout, (size_t)rblocks * 256 * sizeof(unsigned)));
  ms = time_ms([&] { hipLaunchKernelGGL(read_kernel, dim3(rblocks), dim3(256), 0, 0, src, n, rout); }, 10);
  const double read_gbs = (double)n * 16 / (ms * 1e-3) / 1e9;
  const long groups = n * 16 / 4096;
  const uint32_t span = (uint32_t)(groups * 4096 < 0xffffffffL ? groups * 4096 : 0xffffffffL);
  ms = time_ms([&] { hipLaunchKernelGGL(read_dma_kernel<4>, dim3(cus * 2), dim3(256), 0, 0, src, span, groups, rout); }, 10);
  const double read_dma_gbs = (double)groups * 4096 / (ms * 1e-3) / 1e9;
  ms = time_ms([&] { hipLaunchKernelGGL(read_dma_kernel<2>, dim3(cus * 4), dim3(256), 0, 0, src, span, groups, rout); }, 10);
  const double read_dma2_gbs = (double)groups * 4096 / (ms * 1e-3) / 1e9;
  CHECK(hipFree(rout));

  printf("{\"device\": \"%s\", \"cus\": %d, \"clock_mhz\": %d, "
         "\"read_gbs\": %.1f, \"read_lds_dma_4stage_gbs\": %.1f, \"read_lds_dma_2stage_gbs\": %.1f, "
         "\"mfma_bf16_32x32x16_tflops\": %.1f, \"exp2_plus_sub_tops\": %.3f, "
         "\"exp2_tops\": %.3f, \"fma_tops\": %.3f, \"lds_read_tbs\": %.2f, "
         "\"copy_gbs\": %.1f, \"copy_bytes_each_way\": %ld, "
         "\"mfma_mix_2w_tflops\": {\"mfma_only\": %.1f, \"plus_4_fma\": %.1f, "
         "\"plus_1_exp\": %.1f, \"plus_1_lds16\": %.1f, \"plus_4_fma_1_exp_1_lds16\": %.1f, "
         "\"plus_2_lds8_tr\": %.1f, \"plus_4_fma_1_exp_2_lds8_tr\": %.1f, "
         "\"plus_4_fma_1_exp_alternating_lds16_or_2_lds8_tr\": %.1f}, "
         "\"lds_read8_tbs\": %.2f, \"lds_read8_tr_tbs\": %.2f}\n",
         prop.name, cus, prop.clockRate / 1000, read_gbs, read_dma_gbs, read_dma2_gbs, mfma_tflops, exp_sub_rate, exp_rate, fma_rate,
         lds_tbs, copy_gbs, n * 16, mix_pure, mix_v4, mix_x1, mix_l1, mix_all, mix_t1, mix_all_t, mix_alt,
         lds8_tbs, lds8tr_tbs);
  CHECK(hipFree(src));
  CHECK(hipFree(dst));
  CHECK(hipFree(out));
  return 0;
}
