// Internal interface between the C ABI layer and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attnfwd {

// Everything one attention launch needs.  Strides are in elements.
// Dense: sequence `b` starts at b * *_bs.  Varlen: sequence `s` starts at row
// cu_*[s], so the *_bs strides are unused and rows advance by *_ss.
struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  float* o;
  float* lse;  // may be null
  const int32_t* cu_q;  // varlen only
  const int32_t* cu_k;  // varlen only
  // Padded layout (varlen only, may be null): compact row r lives at row
  // row_of[r] of q/k/v/o, and the rows of one sequence are consecutive there,
  // so a sequence starts at row row_of[cu[s]].  The LSE stays indexed by
  // compact row.
  const int32_t* row_of;
  int64_t q_bs, q_ss, q_hs;
  int64_t k_bs, k_ss, k_hs;
  int64_t v_bs, v_ss, v_hs;
  int64_t o_bs, o_ss, o_hs;
  int64_t lse_bs, lse_hs;  // dense: (B, Hq, Sq); varlen: (Hq, Tq) with hs = Tq
  int32_t nseq, hq, hkv, group;
  int32_t sq, sk;    // dense sequence lengths; varlen with single_seq: total_q, total_k
  // Varlen with one sequence and no row map: its offsets are 0 and its lengths
  // total_q / total_k (the cu_seqlens contract), so the kernels take them from
  // sq / sk instead of loading cu_seqlens (one dependent memory round trip
  // less before the first tile).
  int32_t single_seq;
  int32_t n_qb;      // query blocks per (sequence, head) in the grid
  int32_t n_vblk;    // order 4: block slots per head, ceil(total_q / bm) + nseq
  float c;           // |scale| * log2(e): scores enter exp2 in base-2 units
  // Sign of the scale, applied to the Q fragments once per block:
  // q' = (q ^ q_xor) & ~q_clear on each 32-bit word.  scale < 0: q_xor holds
  // the sign bit of every element (exact negation, so c * (-q).k = scale * q.k
  // with c = |scale| log2 e); scale == 0: q_clear = all ones (every score is
  // exactly 0, the same weights as a zero scale); otherwise both 0.  The
  // kernels take the row maximum of the raw scores and multiply it by c, which
  // needs c > 0.  Zero-initialised arguments mean "unchanged".
  uint32_t q_xor;
  uint32_t q_clear;
  int32_t causal;
  int32_t xcd_remap; // 1: spread (sequence, head) rows so each XCD gets a contiguous slice;
                     // 2 (DMA-staged kernel, hq % 8 == 0): sequence-major order, each
                     //   XCD keeping hq/8 fixed heads of the current sequence;
                     // 3 (DMA-staged and pipelined kernels): (sequence, head) units
                     //   dealt to the XCDs, all blocks of a unit in a row (grid
                     //   padded to whole rounds of 8 units)
                     // 4 (DMA-staged kernel, varlen): compact order, one workgroup
                     //   slot per real query block (n_vblk slots per head)
  // Split key ranges (DMA-staged kernel only).  n_split == 1: off.  Otherwise
  // a query block whose key loop has more than split_tiles tiles of split_bn
  // keys is cut into up to n_split even parts; each part writes its
  // normalised partial output and base-2 LSE to part_o / part_lse, and
  // merge_split combines them.
  int32_t n_split;
  int32_t split_tiles;
  int32_t split_bn;
  float* part_o;    // [rows][n_qb][n_split][bm][head_dim]
  float* part_lse;  // [rows][n_qb][n_split][bm]
};

// First q/k/v/o row of varlen sequence `seq` and its lengths.  qs / ks are
// the compact offsets (cu_q[seq], cu_k[seq]); q_row / k_row the storage rows.
struct SeqRows {
  int qs, ks, lq, lk, q_row, k_row;
};
__device__ __forceinline__ SeqRows seq_rows(const AttnArgs& a, int seq) {
  SeqRows r;
  if (a.single_seq) {
    r.qs = r.ks = r.q_row = r.k_row = 0;
    r.lq = a.sq;
    r.lk = a.sk;
    return r;
  }
  r.qs = a.cu_q[seq];
  r.ks = a.cu_k[seq];
  r.lq = a.cu_q[seq + 1] - r.qs;
  r.lk = a.cu_k[seq + 1] - r.ks;
  r.q_row = r.qs;
  r.k_row = r.ks;
  if (a.row_of != nullptr) {
    if (r.lq > 0) r.q_row = a.row_of[r.qs];
    if (r.lk > 0) r.k_row = a.row_of[r.ks];
  }
  return r;
}

// Number of parts a query block with n_kt key tiles is cut into.
__host__ __device__ inline int split_parts(int n_kt, int n_split, int split_tiles) {
  if (n_split <= 1 || n_kt <= split_tiles) return 1;
  const int want = (n_kt + split_tiles - 1) / split_tiles;
  return want < n_split ? want : n_split;
}

// Tile policies: the query block BM = waves * 32 * qcols, key block BN.
struct TilePolicy {
  int waves;   // wavefronts per workgroup
  int qcols;   // 32-query column blocks per wave
  int bn;      // keys per LDS tile
  int kg = 1;  // key groups: waves / kg waves split the queries, kg groups split the keys
  int bm() const { return waves / kg * 32 * qcols; }
};

// Picks the policy for a head_dim and the longest query length.  `override_id`
// (>= 0) forces one of the compiled policies for sweeps.
// `rows` is the number of (sequence, head) pairs of the launch.
bool select_policy(int head_dim, int max_seqlen_q, bool causal, int64_t rows, int override_id,
                   TilePolicy* out, int* policy_id);

// Enqueues one attention launch.  Returns hipSuccess or the launch error.
hipError_t launch_attention(const AttnArgs& a, int head_dim, bool varlen, int policy_id,
                            hipStream_t stream);

// The head_dim 256 part of launch_attention, compiled in its own translation
// unit (attn_kernel_d256.hip) with a different instruction scheduler.
hipError_t launch_attention_d256(const AttnArgs& a, bool varlen, int policy_id, hipStream_t stream);

// Combines the partial outputs of split query blocks (after launch_attention
// with n_split > 1).  bm is the query block of the policy used.
hipError_t launch_merge(const AttnArgs& a, int head_dim, bool varlen, int bm, hipStream_t stream);

// Enqueues the attention backward: D = rowsum(dO * O) into a.part_lse (laid
// out like the LSE), then dQ, then dK / dV.  a.o is the forward output, a.lse
// its natural-log LSE; dout has the layout of q; dq / dk / dv are fp32 with
// the shapes of q / k / v.  n_pairs = query rows * heads, n_kb = key blocks
// of 128 per (sequence, key head).  head_dim 64 or 128.
hipError_t launch_attention_bwd(const AttnArgs& a, int head_dim, bool varlen, const uint16_t* dout,
                                float* dq, float* dk, float* dv, int64_t n_pairs, int n_kb,
                                hipStream_t stream);

// Row gather of up to three tensors sharing one index list.
hipError_t launch_gather(const void* const* src, void* const* dst, int n_tensors,
                         const int32_t* indices, int n_valid, int n_rows_src, int64_t row_bytes,
                         hipStream_t stream);

// Row scatter with zero fill of the rows no index names.  src == nullptr:
// only the zero fill (indexed rows are left untouched).
hipError_t launch_scatter(const void* src, void* dst, const int32_t* indices, int n_valid,
                          int n_rows_total, int64_t row_bytes, hipStream_t stream);

// fp8 (E4M3) attention: q/k/v hold bytes (strides in bytes), a.c includes the
// q and k factors, o_mul = the v factor.  head_dim 64 or 128; bm = queries per
// block, 128 (4 waves, 64-key tiles) or 256 (8 waves, 128-key tiles), with
// a.n_qb counted in blocks of bm.
hipError_t launch_attention_fp8(const AttnArgs& a, int head_dim, bool varlen, float o_mul, int bm,
                                hipStream_t stream);

// Library-owned scratch memory (noalloc.hip): its size, and the current
// device's copy of it (looked up once per device, then cached).
int64_t noalloc_scratch_bytes();
hipError_t noalloc_scratch(void** ptr);

// Debug-mode checks of device-resident preconditions (debug_checks.hip).  The
// checks OR bits into one device status word; debug_status synchronises the
// stream and reads it (0 = consistent, -1 = HIP error).
hipError_t debug_reset(hipStream_t s);
hipError_t debug_check_cu(const int32_t* cu, int n, int total, int max_len, hipStream_t s);
hipError_t debug_check_lens(const int32_t* lens, int n, int max_len, hipStream_t s);
hipError_t debug_check_indices(const int32_t* idx, int n, int n_rows, hipStream_t s);
// idx (n_idx entries) holds consecutive rows within each sequence of cu (n + 1
// offsets): the precondition of the fused padded call.
hipError_t debug_check_runs(const int32_t* idx, int n_idx, const int32_t* cu, int n,
                            hipStream_t s);
int debug_status(hipStream_t s);

// Padding mask (B slots x L rows, nonzero = valid) -> indices of the valid
// rows in row-major order, cu_seqlens (B + 1) and stats = {n_valid,
// max_seqlen}.  indices must hold B * L entries.
hipError_t launch_mask_to_varlen(const uint8_t* mask, int B, int L, int32_t* indices,
                                 int32_t* cu_seqlens, int32_t* stats, hipStream_t stream);

}  // namespace attnfwd
