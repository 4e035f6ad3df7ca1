// Internal interface of the paged-KV attention kernels (decode_kernel.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attnfwd {

struct DecodeArgs {
  const uint16_t* q;           // (tq, hq, D) bf16
  const uint16_t* k_cache;     // (num_pages, page_size, hkv, D) bf16, or E4M3 bytes
  const uint16_t* v_cache;
  const int32_t* block_table;  // (nseq, max_pages)
  const int32_t* seqlens_k;    // (nseq)
  const int32_t* cu_q;         // (nseq + 1)
  float* o;                    // (tq, hq, D)
  float* lse;                  // (hq, tq) natural log, may be null
  float* part_o;               // split only: [nseq][hkv][n_rb][n_split][32][D]
  float* part_lse;             //             [nseq][hkv][n_rb][n_split][32], base 2
  int32_t nseq, tq, hq, hkv, group;
  int32_t num_pages, page_size, max_pages;
  int32_t n_rb;         // 32-row blocks per (sequence, KV head); row r = query * group + head
  int32_t n_split;      // key-range parts per block (1: no split)
  int32_t chunk_tiles;  // 32-key tiles per part
  float c;              // scale * log2(e)
  int32_t causal;
  int32_t order;        // grid order: 1 = KV head fastest, 0 = key part fastest
  int32_t kv_fp8;       // 1: the caches hold E4M3 bytes (dequantised to bf16 in registers)
  float o_mul;          // factor on the output (the v factor of an E4M3 cache; else 1)
};

// Query rows and key tiles of one (sequence, row block).
struct DecodeRange {
  int q0, lq, lk, rows, n_kt;
};

__device__ __forceinline__ DecodeRange decode_range(const DecodeArgs& a, int seq, int rb) {
  DecodeRange d;
  d.q0 = a.cu_q[seq];
  d.lq = a.cu_q[seq + 1] - d.q0;
  d.lk = a.seqlens_k[seq];
  d.rows = d.lq * a.group;
  int kend = d.lk;
  if (a.causal && rb * 32 < d.rows) {
    const int last_q = (min(d.rows, rb * 32 + 32) - 1) / a.group;
    kend = min(d.lk, last_q + d.lk - d.lq + 1);
  }
  if (rb * 32 >= d.rows) d.rows = 0;
  d.n_kt = kend > 0 ? (kend + 31) / 32 : 0;
  return d;
}

__host__ __device__ inline int decode_parts(const DecodeArgs& a, int n_kt) {
  if (a.n_split <= 1) return 1;
  int p = (n_kt + a.chunk_tiles - 1) / a.chunk_tiles;
  if (p > a.n_split) p = a.n_split;
  return p < 1 ? 1 : p;
}

// variant: waves x stages per workgroup (bf16 cache, d=128: 0 = 4x2, 1 = 3x3,
// 2 = 5x2; d=64: 0 = 4x4, 1 = 8x2, 2 = 5x4; E4M3 cache, d=128: 0 = 4x4,
// 1 = 8x2, 2 = 5x4; d=64: 0 = 4x4, 1 = 8x4, 2 = 5x4); < 0 picks the measured
// default.
hipError_t launch_decode(const DecodeArgs& a, int head_dim, int variant, hipStream_t stream);

}  // namespace attnfwd
