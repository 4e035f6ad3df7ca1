// C ABI of the attention library: argument checks, tile-policy choice and
// launch.  Every check runs on the host before anything is enqueued; nothing
// here allocates device memory or synchronises.

#include "../../include/attn_fwd.h"
#include "attn_internal.h"
#include "decode_internal.h"

#include <math.h>
#include <stdlib.h>

#include <algorithm>
#include <initializer_list>

using attnfwd::AttnArgs;
using attnfwd::TilePolicy;

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

bool head_dim_ok(int d) { return d == 32 || d == 64 || d == 128 || d == 256; }

// ATTN_FWD_TILE=<policy id> forces a compiled tile policy (used by tile sweeps).
int tile_override() {
  const char* s = getenv("ATTN_FWD_TILE");
  if (s == nullptr || *s == '\0') return -1;
  char* end = nullptr;
  long v = strtol(s, &end, 10);
  if (end == s || v < 0 || v > 1000) return -1;
  return (int)v;
}

// ATTN_FWD_SPLIT_TILES=<n> forces the key-range split of the DMA-staged
// policies to parts of at most n tiles (used by parity tests of the split path).
int split_override() {
  const char* s = getenv("ATTN_FWD_SPLIT_TILES");
  if (s == nullptr || *s == '\0') return -1;
  char* end = nullptr;
  long v = strtol(s, &end, 10);
  if (end == s || v < 1 || v > 1000000) return -1;
  return (int)v;
}

// Key-range split of long query blocks (DMA-staged policies 11-13, 17, 19).  A
// causal launch with few blocks is bound by its longest block: the last query
// block walks the whole key range while most CUs sit idle.  The plan cuts a
// block's key loop into parts of about the per-CU share of all tiles, so no
// workgroup runs much longer than that share; a merge launch combines parts.
struct SplitPlan {
  int n_split = 1;
  int split_tiles = 0;
  int bn = 64;
  int bm = 0;
};

SplitPlan plan_split(const TilePolicy& pol, int pid, int64_t rows, int n_qb, int max_q,
                     bool causal) {
  SplitPlan sp;
  sp.bm = pol.bm();
  sp.bn = pol.bn;
  if (!(pid >= 11 && pid <= 13) && pid != 17 && pid != 19) return sp;
  const int64_t bm = pol.bm(), bn = pol.bn;
  const int64_t max_tiles = (max_q + bn - 1) / bn;
  int64_t total = 0;  // key tiles summed over the blocks of one (sequence, head)
  for (int64_t qb = 0; qb < n_qb; ++qb) {
    const int64_t keys = causal ? std::min<int64_t>(max_q, (qb + 1) * bm) : max_q;
    total += (keys + bn - 1) / bn;
  }
  total *= rows;
  const int64_t slots = (pid == 13) ? 512 : 256;  // resident workgroups on 256 CUs
  int64_t st = split_override();
  if (st < 1) {
    // Measured: splitting pays only while the blocks alone leave CUs idle
    // (1x8192 causal d=128 with 2 heads: 112 -> 83 us; 1x16384 with 1 head:
    // 213 -> 137 us); with at least one block per slot the extra workgroups,
    // partial stores and merge cost more than the shorter critical path saves
    // (1x2048 with 16 heads: 41 -> 50 us).
    if (rows * n_qb >= slots) return sp;
    const int64_t share = (total + slots - 1) / slots;
    if (max_tiles * 4 <= share * 5) return sp;  // longest block within 25% of the share
    st = std::max<int64_t>(share, 2 * pol.kg);
  }
  const int64_t parts = (max_tiles + st - 1) / st;
  if (parts <= 1) return sp;
  sp.n_split = (int)std::min<int64_t>(parts, 8);
  sp.split_tiles = (int)st;
  return sp;
}

int64_t split_workspace_bytes(const SplitPlan& sp, int64_t rows, int n_qb, int head_dim) {
  if (sp.n_split <= 1) return 0;
  return rows * n_qb * sp.n_split * sp.bm * (int64_t)(head_dim + 1) * 4;
}

// scale * log2(e), the factor that turns scores into base-2 exponents.
float base2_factor(float scale) { return (float)((double)scale * 1.4426950408889634074); }

// The forward kernels take the row maximum of the raw scores before
// multiplying by c, so they need c > 0.  Any finite scale reaches that form
// exactly: c = |scale| log2(e) (times the fp8 factors `extra`), and the sign
// goes onto Q once per block -- a negative scale negates every Q element (a
// sign-bit flip, exact in bf16 and E4M3), a zero scale clears Q (every score is
// then exactly 0, the uniform weights a zero scale gives).  sign_bits holds the
// sign bit of every element of a 32-bit word (0x80008000 for bf16, 0x80808080
// for E4M3).
void set_forward_scale(AttnArgs& a, float scale, double extra, uint32_t sign_bits) {
  const double mag = scale == 0.f ? 1.0 : fabs((double)scale);
  a.c = (float)(mag * extra * 1.4426950408889634074);
  a.q_xor = scale < 0.f ? sign_bits : 0u;
  a.q_clear = scale == 0.f ? 0xffffffffu : 0u;
}

attn_status_t check_common(int32_t hq, int32_t hkv, int32_t d, float scale) {
  if (hq < 0 || hkv < 0) return ATTN_ERR_SHAPE;
  if (!head_dim_ok(d)) return ATTN_ERR_UNSUPPORTED;
  if (!isfinite(scale)) return ATTN_ERR_UNSUPPORTED;
  if (hq > 0 && (hkv <= 0 || hq % hkv != 0)) return ATTN_ERR_SHAPE;
  return ATTN_OK;
}

// Tile loads address one sequence's rows through 32-bit buffer offsets.
bool span_fits(int64_t rows, int64_t row_stride_elems) {
  return rows * row_stride_elems * 2 < (1LL << 32);
}

// ATTN_FWD_ORDER=<n> forces the workgroup order of a launch (tests comparing
// orders bit for bit): 1 head-remapped block-major, 2 sequence-major, 3
// unit-major, 4 compact.  A launch the forced order cannot serve returns
// ATTN_ERR_UNSUPPORTED.
int order_override() {
  const char* s = getenv("ATTN_FWD_ORDER");
  if (s == nullptr || *s == '\0') return -1;
  char* end = nullptr;
  long v = strtol(s, &end, 10);
  if (end == s || v < 0 || v > 4) return -1;
  return (int)v;
}

// The launch plan of one forward call: tile policy, workgroup order, split
// parts.  Fills the plan fields of `a` (n_qb, xcd_remap, n_vblk, n_split,
// split_tiles, split_bn, part_o, part_lse).  Pure host computation.
attn_status_t plan_launch(AttnArgs& a, int d, bool varlen, int max_q, void* ws, int64_t ws_bytes,
                          int* pid_out, int* bm_out) {
  TilePolicy pol;
  int pid;
  const int64_t rows = (int64_t)a.nseq * a.hq;
  if (!attnfwd::select_policy(d, max_q, a.causal != 0, rows, tile_override(), &pol, &pid))
    return ATTN_ERR_UNSUPPORTED;
  a.n_qb = (max_q + pol.bm() - 1) / pol.bm();
  a.xcd_remap = (rows % 8 == 0) ? 1 : 0;
  // Several sequences (or a batch) on the DMA-staged kernel: sequence-major
  // workgroup order, so the workgroups an XCD runs at once share a few heads'
  // K/V in its L2 (a 64K-token pack of 17 sequences: 2072 -> 1406 us).
  const bool dma_kernel = (pid >= 11 && pid <= 13) || pid >= 17;
  const bool pipe_kernel = pid >= 14 && pid <= 16;
  if (dma_kernel && a.nseq > 1 && a.hq % 8 == 0) a.xcd_remap = 2;
  // Otherwise, on several sequences: unit-major order, every block of one
  // (sequence, head) on one XCD in a row (ViT batch, 149 x 12 heads, d=64:
  // 770 -> 712 us).  Not with split parts (their plan needs the block order).
  const bool unit_major = (dma_kernel || pipe_kernel) && a.nseq > 1 && a.xcd_remap != 2;
  a.n_split = 1;
  const SplitPlan sp = plan_split(pol, pid, rows, a.n_qb, max_q, a.causal != 0);
  const int64_t need = split_workspace_bytes(sp, rows, a.n_qb, d);
  const bool split = need > 0 && ws_bytes >= need;
  if (unit_major && !split) a.xcd_remap = 3;
  if (split) {
    a.n_split = sp.n_split;
    a.split_tiles = sp.split_tiles;
    a.split_bn = sp.bn;
    a.part_o = static_cast<float*>(ws);
    a.part_lse = ws ? a.part_o + rows * a.n_qb * sp.n_split * sp.bm * d : nullptr;
  }
  // A pack whose longest sequence is far above the rest (one long sequence
  // with many short ones): the (sequence, head) x longest-block-count grid is
  // then mostly workgroups with no block, each holding a CU slot while it
  // reads cu_seqlens (1 x 8192 + 64 x 128, 16 heads: 383 us against 262 for
  // the long sequence alone).  Compact order instead: sequence s owns block
  // slots [cu_q[s] / bm + s, ...), at most ceil(total_q / bm) + nseq per head.
  const int64_t bm = pol.bm();
  const int64_t nv = (a.lse_hs + bm - 1) / bm + a.nseq;  // lse_hs: compact rows
  const bool compact_ok = varlen && dma_kernel && a.n_split == 1 &&
                          (int64_t)a.hq * nv <= 0x7fffffffLL;
  if (compact_ok && a.nseq > 1 && rows * a.n_qb >= 4 * (int64_t)a.hq * nv) a.xcd_remap = 4;
  const int forced = order_override();
  if (forced >= 0) {
    // 1 needs a bijective head remap (rows % 8 == 0); 2 and 3 exist in the
    // DMA-staged kernel (3 also in the pipelined one) and 2 needs hq % 8 == 0;
    // 3 and 4 take no split parts; 4 is varlen only.
    const bool ok = forced == 0 || (forced == 1 && rows % 8 == 0) ||
                    (forced == 2 && dma_kernel && a.hq % 8 == 0) ||
                    (forced == 3 && (dma_kernel || pipe_kernel) && a.n_split == 1) ||
                    (forced == 4 && compact_ok);
    if (!ok) return ATTN_ERR_UNSUPPORTED;
    a.xcd_remap = forced;
  }
  if (a.xcd_remap == 4) a.n_vblk = (int32_t)nv;
  if (rows * a.n_qb * a.n_split > 0x7fffffffLL) return ATTN_ERR_SHAPE;
  *pid_out = pid;
  *bm_out = (int)bm;
  return ATTN_OK;
}

attn_status_t launch(AttnArgs& a, int d, bool varlen, int max_q, void* ws, int64_t ws_bytes,
                     hipStream_t stream) {
  int pid = 0, bm = 0;
  const attn_status_t st = plan_launch(a, d, varlen, max_q, ws, ws != nullptr ? ws_bytes : 0,
                                       &pid, &bm);
  if (st != ATTN_OK) return st;
  hipError_t e = attnfwd::launch_attention(a, d, varlen, pid, stream);
  if (e == hipSuccess && a.n_split > 1) e = attnfwd::launch_merge(a, d, varlen, bm, stream);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

attn_status_t check_workspace(const void* ws, int64_t ws_bytes) {
  if (ws_bytes < 0) return ATTN_ERR_SHAPE;
  if (ws != nullptr && !aligned16(ws)) return ATTN_ERR_ALIGN;
  return ATTN_OK;
}

// Shared checks and launch of the two backward entry points.  `a` carries the
// layout; rows_q is the number of query rows (packed or batch * seqlen_q).
attn_status_t launch_bwd(AttnArgs& a, int d, bool varlen, int max_q, int max_k, int64_t rows_q,
                         const void* dout, float* dq, float* dk, float* dv, void* ws,
                         int64_t ws_bytes, hipStream_t stream) {
  if (ws_bytes < rows_q * a.hq * 4) return ATTN_ERR_SHAPE;
  a.part_lse = static_cast<float*>(ws);
  a.n_qb = (max_q + 127) / 128;
  const int n_kb = (max_k + 127) / 128;
  const hipError_t e = attnfwd::launch_attention_bwd(a, d, varlen, static_cast<const uint16_t*>(dout),
                                                     dq, dk, dv, rows_q * a.hq, n_kb, stream);
  return e == hipSuccess ? ATTN_OK : (e == hipErrorInvalidConfiguration ? ATTN_ERR_SHAPE : ATTN_ERR_HIP);
}

attn_status_t check_bwd_ptrs(const void* q, const void* k, const void* v, const float* out,
                             const void* dout, const float* lse, float* dq, float* dk, float* dv,
                             void* ws) {
  if (!q || !k || !v || !out || !dout || !lse || !dq || !dk || !dv || !ws) return ATTN_ERR_NULL;
  const void* p16[] = {q, k, v, out, dout, dq, dk, dv, ws};
  for (const void* p : p16)
    if (!aligned16(p)) return ATTN_ERR_ALIGN;
  if (!aligned4(lse)) return ATTN_ERR_ALIGN;
  return ATTN_OK;
}


// ---- paged KV cache (decode_kernel.hip)

// ATTN_PAGED_CHUNK_TILES=<n> forces key-range parts of n 32-key tiles (tests).
int paged_chunk_override() {
  const char* s = getenv("ATTN_PAGED_CHUNK_TILES");
  if (s == nullptr || *s == '\0') return -1;
  char* end = nullptr;
  long v = strtol(s, &end, 10);
  if (end == s || v < 1 || v > 1000000) return -1;
  return (int)v;
}

// ATTN_PAGED_VARIANT=<0|1|2|3> picks the waves x stages layout (sweeps).
int paged_variant() {
  const char* s = getenv("ATTN_PAGED_VARIANT");
  if (s == nullptr || *s < '0' || *s > '3' || s[1] != '\0') return -1;
  return *s - '0';
}

// ATTN_PAGED_ORDER=<0|1> picks the grid order (sweeps; default 1).
int paged_order() {
  const char* s = getenv("ATTN_PAGED_ORDER");
  return (s != nullptr && s[0] == '0' && s[1] == '\0') ? 0 : 1;
}

constexpr int64_t kPagedTargetWorkgroups = 256;
// A split plan has fewer than 2 * kPagedTargetWorkgroups slots of 32 rows x
// (head_dim + 1) floats; the no-allocation entry point's static array holds
// any of them at the largest head_dim.
static_assert(2 * kPagedTargetWorkgroups * 32 * (256 + 1) * 4 <= ATTN_NOALLOC_SCRATCH_BYTES,
              "every default paged plan must fit the no-allocation scratch");

struct PagedPlan {
  int n_rb = 0;
  int n_split = 1;
  int chunk_tiles = 0;
};

// Row blocks of 32 (query, head-of-group) pairs, and the key-range split: the
// launch has nseq * hkv * n_rb workgroups before splitting; parts are added
// until about 256 workgroups (one per CU: each fills the CU's LDS) exist,
// keeping at least 8 tiles (2 per wave) in a part.  Fewer, longer parts
// stream faster than more rounds of short ones: each workgroup pays its own
// start (Q, page table, first tiles in flight) and merge, and the last round
// ends ragged (measured with the caches evicted: 32 sequences of 4-8k keys
// 178 -> 166 us, 8 x 32k keys 216 -> 197 us, E4M3 caches -20 %, against
// about 1024 workgroups).
PagedPlan plan_paged(int nseq, int max_q, int max_k, int group, int hkv) {
  PagedPlan p;
  p.n_rb = (int)(((int64_t)max_q * group + 31) / 32);
  const int n_kt = (max_k + 31) / 32;
  const int64_t base = (int64_t)nseq * hkv * p.n_rb;
  if (n_kt <= 0 || base <= 0) return p;
  int parts;
  const int forced = paged_chunk_override();
  if (forced > 0) {
    parts = (n_kt + forced - 1) / forced;
  } else {
    const int64_t want = (kPagedTargetWorkgroups + base - 1) / base;
    parts = (int)std::min<int64_t>(want, (n_kt + 7) / 8);
    parts = std::min(parts, 64);
  }
  if (parts <= 1) return p;
  p.chunk_tiles = (n_kt + parts - 1) / parts;
  p.n_split = (n_kt + p.chunk_tiles - 1) / p.chunk_tiles;
  if (p.n_split <= 1) p.n_split = 1;
  return p;
}

int64_t paged_workspace_bytes(const PagedPlan& p, int nseq, int hkv, int d) {
  if (p.n_split <= 1) return 0;
  return (int64_t)nseq * hkv * p.n_rb * p.n_split * 32 * (int64_t)(d + 1) * 4;
}


attn_status_t check_fp8(int32_t hq, int32_t hkv, int32_t d, float scale, float qs, float ks,
                        float vs) {
  attn_status_t st = check_common(hq, hkv, d, scale);
  if (st != ATTN_OK) return st;
  if (d != 32 && d != 64 && d != 128 && d != 256) return ATTN_ERR_UNSUPPORTED;
  for (float f : {qs, ks, vs})
    if (!(f > 0.f) || !isfinite(f)) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

// ATTN_FP8_TILE=128|256 forces the fp8 query block (sweeps and tests).
int fp8_tile_override() {
  const char* s = getenv("ATTN_FP8_TILE");
  if (s == nullptr || *s == '\0') return -1;
  const long v = strtol(s, nullptr, 10);
  return (v == 128 || v == 256) ? (int)v : -1;
}

attn_status_t launch_fp8(AttnArgs& a, int d, bool varlen, int max_q, float scale, float qs,
                         float ks, float vs, hipStream_t stream) {
  set_forward_scale(a, scale, (double)qs * ks, 0x80808080u);
  // 128-query blocks (4 waves, 64-key tiles, 150 VGPRs: three workgroups per
  // CU).  256-query blocks (8 waves, 128-key tiles: K/V tiles shared by twice
  // the queries, half the barriers and row-maximum passes per key, but 187
  // VGPRs and one workgroup per CU) measured 10-11 % slower on 1x4096 causal
  // and 4x4096 non-causal, and from 2 % faster to 9 % slower on 1x8192 causal
  // depending on the box; they stay selectable with ATTN_FP8_TILE=256.
  const int64_t rows = (int64_t)a.nseq * a.hq;
  int bm = 128;
  if (fp8_tile_override() > 0) bm = fp8_tile_override();
  if (d == 256 && bm != 128) return ATTN_ERR_UNSUPPORTED;  // 256-query blocks: head_dim <= 128
  a.n_qb = (max_q + bm - 1) / bm;
  a.xcd_remap = (rows % 8 == 0) ? 1 : 0;
  const hipError_t e = attnfwd::launch_attention_fp8(a, d, varlen, vs, bm, stream);
  return e == hipSuccess ? ATTN_OK : (e == hipErrorInvalidConfiguration ? ATTN_ERR_SHAPE : ATTN_ERR_HIP);
}

// ATTN_FWD_DEBUG=1 (any value but 0) checks the device-resident preconditions
// (cu_seqlens, indices, seqlens_k) with small kernels before the real work and
// returns ATTN_ERR_SHAPE when one fails; this mode synchronises the stream.
bool debug_mode() {
  const char* s = getenv("ATTN_FWD_DEBUG");
  return s != nullptr && *s != '\0' && !(s[0] == '0' && s[1] == '\0');
}

struct DebugCheck {
  const int32_t* cu = nullptr;  // cu-style offsets: n + 1 entries
  int n = -1, total = 0, max_len = -1;
  const int32_t* lens = nullptr;  // per-sequence lengths: n_lens entries
  int n_lens = 0, lens_max = 0;
  const int32_t* idx = nullptr;  // indices: n_idx entries
  int n_idx = 0, idx_rows = -1;
  const int32_t* runs_cu = nullptr;  // with idx: idx consecutive within each of n_runs sequences
  int n_runs = 0;
};

attn_status_t run_debug(std::initializer_list<DebugCheck> checks, hipStream_t s) {
  if (!debug_mode()) return ATTN_OK;
  if (attnfwd::debug_reset(s) != hipSuccess) return ATTN_ERR_HIP;
  for (const DebugCheck& c : checks) {
    if (c.cu && attnfwd::debug_check_cu(c.cu, c.n, c.total, c.max_len, s) != hipSuccess)
      return ATTN_ERR_HIP;
    if (c.lens && attnfwd::debug_check_lens(c.lens, c.n_lens, c.lens_max, s) != hipSuccess)
      return ATTN_ERR_HIP;
    if (c.idx && attnfwd::debug_check_indices(c.idx, c.n_idx, c.idx_rows, s) != hipSuccess)
      return ATTN_ERR_HIP;
    if (c.idx && c.runs_cu &&
        attnfwd::debug_check_runs(c.idx, c.n_idx, c.runs_cu, c.n_runs, s) != hipSuccess)
      return ATTN_ERR_HIP;
  }
  const int st = attnfwd::debug_status(s);
  return st == 0 ? ATTN_OK : (st < 0 ? ATTN_ERR_HIP : ATTN_ERR_SHAPE);
}

DebugCheck cu_check(const int32_t* cu, int n, int total, int max_len) {
  DebugCheck c;
  c.cu = cu;
  c.n = n;
  c.total = total;
  c.max_len = max_len;
  return c;
}

DebugCheck idx_check(const int32_t* idx, int n, int rows) {
  DebugCheck c;
  c.idx = idx;
  c.n_idx = n;
  c.idx_rows = rows;
  return c;
}

DebugCheck runs_check(const int32_t* idx, int n_idx, const int32_t* cu, int n) {
  DebugCheck c;
  c.idx = idx;
  c.n_idx = n_idx;
  c.runs_cu = cu;
  c.n_runs = n;
  return c;
}

DebugCheck lens_check(const int32_t* lens, int n, int max_len) {
  DebugCheck c;
  c.lens = lens;
  c.n_lens = n;
  c.lens_max = max_len;
  return c;
}


attn_status_t paged_impl(const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* cu_seqlens_q, const int32_t* seqlens_k,
                         const int32_t* block_table, int32_t num_seqs, int32_t total_q,
                         int32_t num_pages, int32_t page_size, int32_t max_pages_per_seq,
                         int32_t num_heads_q, int32_t num_heads_k, int32_t head_dim,
                         int32_t max_seqlen_q, int32_t max_seqlen_k, float scale, int32_t causal,
                         float* out, float* lse, void* workspace, int64_t workspace_bytes,
                         bool kv_fp8, float k_scale, float v_scale, void* stream,
                         bool no_alloc = false) {
  if (num_seqs < 0 || total_q < 0 || num_pages < 0 || max_pages_per_seq < 0 ||
      max_seqlen_q < 0 || max_seqlen_k < 0)
    return ATTN_ERR_SHAPE;
  attn_status_t st = check_common(num_heads_q, num_heads_k, head_dim, scale);
  if (st != ATTN_OK) return st;
  if (!head_dim_ok(head_dim)) return ATTN_ERR_UNSUPPORTED;
  if (page_size < 16 || page_size % 16 != 0) return ATTN_ERR_UNSUPPORTED;
  if (kv_fp8)
    for (float f : {k_scale, v_scale})
      if (!(f > 0.f) || !isfinite(f)) return ATTN_ERR_UNSUPPORTED;
  st = check_workspace(workspace, workspace_bytes);
  if (st != ATTN_OK) return st;
  if (num_seqs == 0 || total_q == 0 || num_heads_q == 0) return ATTN_OK;
  if (max_seqlen_q == 0) return ATTN_ERR_SHAPE;
  if ((int64_t)max_seqlen_k > (int64_t)max_pages_per_seq * page_size) return ATTN_ERR_SHAPE;
  if (q == nullptr || out == nullptr || cu_seqlens_q == nullptr || seqlens_k == nullptr)
    return ATTN_ERR_NULL;
  if (max_seqlen_k > 0 && (k_cache == nullptr || v_cache == nullptr || block_table == nullptr))
    return ATTN_ERR_NULL;
  if (!aligned16(q) || !aligned16(out) ||
      (max_seqlen_k > 0 && (!aligned16(k_cache) || !aligned16(v_cache))))
    return ATTN_ERR_ALIGN;
  if (!aligned4(cu_seqlens_q) || !aligned4(seqlens_k) || (block_table && !aligned4(block_table)) ||
      (lse && !aligned4(lse)))
    return ATTN_ERR_ALIGN;
  const int64_t page_bytes = (int64_t)page_size * num_heads_k * head_dim * (kv_fp8 ? 1 : 2);
  if (page_bytes >= (1LL << 32)) return ATTN_ERR_SHAPE;
  attnfwd::DecodeArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k_cache = static_cast<const uint16_t*>(k_cache);
  a.v_cache = static_cast<const uint16_t*>(v_cache);
  a.block_table = block_table;
  a.seqlens_k = seqlens_k;
  a.cu_q = cu_seqlens_q;
  a.o = out;
  a.lse = lse;
  a.nseq = num_seqs;
  a.tq = total_q;
  a.hq = num_heads_q;
  a.hkv = num_heads_k;
  a.group = num_heads_q / num_heads_k;
  a.num_pages = num_pages;
  a.page_size = page_size;
  a.max_pages = max_pages_per_seq;
  a.c = kv_fp8 ? (float)((double)scale * k_scale * 1.4426950408889634074) : base2_factor(scale);
  a.causal = causal ? 1 : 0;
  a.order = paged_order();
  a.kv_fp8 = kv_fp8 ? 1 : 0;
  a.o_mul = kv_fp8 ? v_scale : 1.f;
  {
    const attn_status_t dst_ = run_debug({cu_check(cu_seqlens_q, num_seqs, total_q, max_seqlen_q),
                                          lens_check(seqlens_k, num_seqs, max_seqlen_k)},
                                         static_cast<hipStream_t>(stream));
    if (dst_ != ATTN_OK) return dst_;
  }
  const int max_q = max_seqlen_q < total_q ? max_seqlen_q : total_q;
  const PagedPlan p = plan_paged(num_seqs, max_q, max_seqlen_k, a.group, num_heads_k);
  a.n_rb = p.n_rb;
  a.n_split = 1;
  a.chunk_tiles = 0;
  const int64_t need = paged_workspace_bytes(p, num_seqs, num_heads_k, head_dim);
  if (no_alloc) {
    // the library's own scratch array instead of a caller workspace
    if (need > attnfwd::noalloc_scratch_bytes()) return ATTN_ERR_SCRATCH;
    if (attnfwd::noalloc_scratch(&workspace) != hipSuccess) return ATTN_ERR_HIP;
    workspace_bytes = attnfwd::noalloc_scratch_bytes();
  }
  if (need > 0 && workspace != nullptr && workspace_bytes >= need) {
    a.n_split = p.n_split;
    a.chunk_tiles = p.chunk_tiles;
    a.part_o = static_cast<float*>(workspace);
    a.part_lse = a.part_o + (int64_t)num_seqs * num_heads_k * p.n_rb * p.n_split * 32 * head_dim;
  }
  const hipError_t e =
      attnfwd::launch_decode(a, head_dim, paged_variant(), static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : (e == hipErrorInvalidConfiguration ? ATTN_ERR_SHAPE : ATTN_ERR_HIP);
}

}  // namespace

extern "C" {

attn_status_t attn_fwd_varlen_ws(const void* q, const void* k, const void* v,
                                 const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                 int32_t num_seqs, int32_t total_q, int32_t total_k,
                                 int32_t num_heads_q, int32_t num_heads_k, int32_t head_dim,
                                 int32_t max_seqlen, float scale, int32_t causal, float* out,
                                 float* lse, void* workspace, int64_t workspace_bytes,
                                 void* stream) {
  if (num_seqs < 0 || total_q < 0 || total_k < 0 || max_seqlen < 0) return ATTN_ERR_SHAPE;
  attn_status_t st = check_common(num_heads_q, num_heads_k, head_dim, scale);
  if (st != ATTN_OK) return st;
  st = check_workspace(workspace, workspace_bytes);
  if (st != ATTN_OK) return st;
  if (num_seqs == 0 || total_q == 0 || num_heads_q == 0) return ATTN_OK;
  if (max_seqlen == 0) return ATTN_ERR_SHAPE;  // some sequence has queries
  if (q == nullptr || out == nullptr || cu_seqlens_q == nullptr || cu_seqlens_k == nullptr)
    return ATTN_ERR_NULL;
  if (total_k > 0 && (k == nullptr || v == nullptr)) return ATTN_ERR_NULL;
  if (!aligned16(q) || !aligned16(out) || (total_k > 0 && (!aligned16(k) || !aligned16(v))))
    return ATTN_ERR_ALIGN;
  if (!aligned4(cu_seqlens_q) || !aligned4(cu_seqlens_k) || (lse && !aligned4(lse)))
    return ATTN_ERR_ALIGN;

  AttnArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = out;
  a.lse = lse;
  a.cu_q = cu_seqlens_q;
  a.cu_k = cu_seqlens_k;
  a.q_ss = (int64_t)num_heads_q * head_dim;
  a.q_hs = head_dim;
  a.k_ss = (int64_t)num_heads_k * head_dim;
  a.k_hs = head_dim;
  a.v_ss = a.k_ss;
  a.v_hs = head_dim;
  a.o_ss = a.q_ss;
  a.o_hs = head_dim;
  a.lse_hs = total_q;
  a.nseq = num_seqs;
  a.hq = num_heads_q;
  a.hkv = num_heads_k;
  a.group = num_heads_q / num_heads_k;
  set_forward_scale(a, scale, 1.0, 0x80008000u);
  a.causal = causal ? 1 : 0;
  if (!span_fits(total_q, a.q_ss) || !span_fits(total_k, a.k_ss)) return ATTN_ERR_SHAPE;
  st = run_debug({cu_check(cu_seqlens_q, num_seqs, total_q, max_seqlen),
                  cu_check(cu_seqlens_k, num_seqs, total_k, -1)},
                 static_cast<hipStream_t>(stream));
  if (st != ATTN_OK) return st;
  if (num_seqs == 1) {  // offsets 0, lengths total_q / total_k by the cu_seqlens contract
    a.single_seq = 1;
    a.sq = total_q;
    a.sk = total_k;
  }
  const int max_q = max_seqlen < total_q ? max_seqlen : total_q;
  return launch(a, head_dim, true, max_q, workspace, workspace_bytes,
                static_cast<hipStream_t>(stream));
}

attn_status_t attn_fwd_varlen(const void* q, const void* k, const void* v,
                              const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                              int32_t num_seqs, int32_t total_q, int32_t total_k,
                              int32_t num_heads_q, int32_t num_heads_k, int32_t head_dim,
                              int32_t max_seqlen, float scale, int32_t causal, float* out,
                              float* lse, void* stream) {
  return attn_fwd_varlen_ws(q, k, v, cu_seqlens_q, cu_seqlens_k, num_seqs, total_q, total_k,
                            num_heads_q, num_heads_k, head_dim, max_seqlen, scale, causal, out,
                            lse, nullptr, 0, stream);
}

attn_status_t attn_fwd_dense_ws(const void* q, const void* k, const void* v, int32_t batch,
                                int32_t seqlen_q, int32_t seqlen_k, int32_t num_heads_q,
                                int32_t num_heads_k, int32_t head_dim, const int64_t* strides,
                                float scale, int32_t causal, float* out, float* lse,
                                void* workspace, int64_t workspace_bytes, void* stream) {
  if (batch < 0 || seqlen_q < 0 || seqlen_k < 0) return ATTN_ERR_SHAPE;
  attn_status_t st = check_common(num_heads_q, num_heads_k, head_dim, scale);
  if (st != ATTN_OK) return st;
  st = check_workspace(workspace, workspace_bytes);
  if (st != ATTN_OK) return st;
  if (batch == 0 || seqlen_q == 0 || num_heads_q == 0) return ATTN_OK;
  if (q == nullptr || out == nullptr) return ATTN_ERR_NULL;
  if (seqlen_k > 0 && (k == nullptr || v == nullptr)) return ATTN_ERR_NULL;
  if (!aligned16(q) || !aligned16(out) || (seqlen_k > 0 && (!aligned16(k) || !aligned16(v))))
    return ATTN_ERR_ALIGN;
  if (lse && !aligned4(lse)) return ATTN_ERR_ALIGN;

  AttnArgs a{};
  const int64_t d = head_dim;
  if (strides == nullptr) {
    a.q_hs = d;
    a.q_ss = num_heads_q * d;
    a.q_bs = a.q_ss * seqlen_q;
    a.k_hs = d;
    a.k_ss = num_heads_k * d;
    a.k_bs = a.k_ss * seqlen_k;
    a.v_hs = a.k_hs;
    a.v_ss = a.k_ss;
    a.v_bs = a.k_bs;
    a.o_hs = d;
    a.o_ss = num_heads_q * d;
    a.o_bs = a.o_ss * seqlen_q;
  } else {
    for (int i = 0; i < 12; ++i) {
      if (strides[i] < 0) return ATTN_ERR_SHAPE;
      if (i < 9 && strides[i] % 8 != 0) return ATTN_ERR_ALIGN;
      if (i >= 9 && strides[i] % 4 != 0) return ATTN_ERR_ALIGN;
    }
    a.q_bs = strides[0]; a.q_ss = strides[1]; a.q_hs = strides[2];
    a.k_bs = strides[3]; a.k_ss = strides[4]; a.k_hs = strides[5];
    a.v_bs = strides[6]; a.v_ss = strides[7]; a.v_hs = strides[8];
    a.o_bs = strides[9]; a.o_ss = strides[10]; a.o_hs = strides[11];
  }
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = out;
  a.lse = lse;
  a.lse_hs = seqlen_q;
  a.lse_bs = (int64_t)num_heads_q * seqlen_q;
  a.nseq = batch;
  a.hq = num_heads_q;
  a.hkv = num_heads_k;
  a.group = num_heads_q / num_heads_k;
  a.sq = seqlen_q;
  a.sk = seqlen_k;
  set_forward_scale(a, scale, 1.0, 0x80008000u);
  a.causal = causal ? 1 : 0;
  if (!span_fits(seqlen_q, a.q_ss) || !span_fits(seqlen_k, a.k_ss) || !span_fits(seqlen_k, a.v_ss))
    return ATTN_ERR_SHAPE;
  return launch(a, head_dim, false, seqlen_q, workspace, workspace_bytes,
                static_cast<hipStream_t>(stream));
}

attn_status_t attn_fwd_dense(const void* q, const void* k, const void* v, int32_t batch,
                             int32_t seqlen_q, int32_t seqlen_k, int32_t num_heads_q,
                             int32_t num_heads_k, int32_t head_dim, const int64_t* strides,
                             float scale, int32_t causal, float* out, float* lse, void* stream) {
  return attn_fwd_dense_ws(q, k, v, batch, seqlen_q, seqlen_k, num_heads_q, num_heads_k, head_dim,
                           strides, scale, causal, out, lse, nullptr, 0, stream);
}

int64_t attn_fwd_workspace_bytes(int32_t num_seqs, int32_t max_seqlen, int32_t num_heads_q,
                                 int32_t head_dim, int32_t causal) {
  if (num_seqs <= 0 || max_seqlen <= 0 || num_heads_q <= 0 || !head_dim_ok(head_dim)) return 0;
  TilePolicy pol;
  int pid;
  const int64_t rows = (int64_t)num_seqs * num_heads_q;
  if (!attnfwd::select_policy(head_dim, max_seqlen, causal != 0, rows, tile_override(), &pol, &pid))
    return 0;
  const int n_qb = (max_seqlen + pol.bm() - 1) / pol.bm();
  const SplitPlan sp = plan_split(pol, pid, rows, n_qb, max_seqlen, causal != 0);
  return split_workspace_bytes(sp, rows, n_qb, head_dim);
}

attn_status_t attn_fwd_launch_plan(int32_t varlen, int32_t num_seqs, int32_t total_q,
                                   int32_t max_seqlen, int32_t num_heads_q, int32_t head_dim,
                                   int32_t causal, int64_t workspace_bytes, int32_t* plan) {
  if (plan == nullptr) return ATTN_ERR_NULL;
  if (num_seqs <= 0 || total_q <= 0 || max_seqlen <= 0 || num_heads_q <= 0 || workspace_bytes < 0)
    return ATTN_ERR_SHAPE;
  if (!head_dim_ok(head_dim)) return ATTN_ERR_UNSUPPORTED;
  AttnArgs a{};
  a.nseq = num_seqs;
  a.hq = num_heads_q;
  a.causal = causal ? 1 : 0;
  a.lse_hs = varlen ? total_q : max_seqlen;
  const int max_q = varlen ? std::min(max_seqlen, total_q) : max_seqlen;
  int pid = 0, bm = 0;
  const attn_status_t st = plan_launch(a, head_dim, varlen != 0, max_q, nullptr, workspace_bytes,
                                       &pid, &bm);
  if (st != ATTN_OK) return st;
  plan[0] = pid;
  plan[1] = a.xcd_remap;
  plan[2] = a.n_split;
  plan[3] = bm;
  return ATTN_OK;
}

int32_t attn_fwd_tile_policy_compiled(int32_t policy, int32_t head_dim) {
  if (policy < 0 || !head_dim_ok(head_dim)) return 0;
  TilePolicy pol;
  int pid;
  return attnfwd::select_policy(head_dim, 1024, true, 1, policy, &pol, &pid) ? 1 : 0;
}

attn_status_t attn_fwd_padded(const void* q, const void* k, const void* v,
                              const int32_t* indices, const int32_t* cu_seqlens, int32_t num_seqs,
                              int32_t n_valid, int32_t n_rows, int32_t num_heads_q,
                              int32_t num_heads_k, int32_t head_dim, int32_t max_seqlen,
                              float scale, int32_t causal, float* out, float* lse, void* stream) {
  if (num_seqs < 0 || n_valid < 0 || n_rows < 0 || max_seqlen < 0) return ATTN_ERR_SHAPE;
  if (n_valid > n_rows) return ATTN_ERR_SHAPE;
  attn_status_t st = check_common(num_heads_q, num_heads_k, head_dim, scale);
  if (st != ATTN_OK) return st;
  if (n_rows == 0 || num_heads_q == 0) return ATTN_OK;
  if (out == nullptr) return ATTN_ERR_NULL;
  if (!aligned16(out)) return ATTN_ERR_ALIGN;
  const bool work = n_valid > 0 && num_seqs > 0;
  if (work) {
    if (max_seqlen == 0) return ATTN_ERR_SHAPE;
    if (q == nullptr || k == nullptr || v == nullptr || indices == nullptr || cu_seqlens == nullptr)
      return ATTN_ERR_NULL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v)) return ATTN_ERR_ALIGN;
    if (!aligned4(indices) || !aligned4(cu_seqlens) || (lse && !aligned4(lse)))
      return ATTN_ERR_ALIGN;
  } else if (n_valid > 0 && (indices == nullptr || !aligned4(indices))) {
    return indices == nullptr ? ATTN_ERR_NULL : ATTN_ERR_ALIGN;
  }
  const int64_t out_row_bytes = (int64_t)num_heads_q * head_dim * 4;
  if ((int64_t)n_rows * (out_row_bytes / 16) >= (1LL << 31)) return ATTN_ERR_SHAPE;
  AttnArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = out;
  a.lse = lse;
  a.cu_q = cu_seqlens;
  a.cu_k = cu_seqlens;
  a.row_of = indices;
  a.q_ss = (int64_t)num_heads_q * head_dim;
  a.q_hs = head_dim;
  a.k_ss = (int64_t)num_heads_k * head_dim;
  a.k_hs = head_dim;
  a.v_ss = a.k_ss;
  a.v_hs = head_dim;
  a.o_ss = a.q_ss;
  a.o_hs = head_dim;
  a.lse_hs = n_valid;
  a.nseq = num_seqs;
  a.hq = num_heads_q;
  a.hkv = num_heads_k;
  a.group = num_heads_k > 0 ? num_heads_q / num_heads_k : 1;
  set_forward_scale(a, scale, 1.0, 0x80008000u);
  a.causal = causal ? 1 : 0;
  if (!span_fits(n_rows, a.q_ss) || !span_fits(n_rows, a.k_ss)) return ATTN_ERR_SHAPE;
  if (n_valid > 0) {
    const attn_status_t dst_ = run_debug(
        {idx_check(indices, n_valid, n_rows),
         cu_check(cu_seqlens, work ? num_seqs : -1, n_valid, max_seqlen),
         runs_check(indices, n_valid, cu_seqlens, work ? num_seqs : 0)},
        static_cast<hipStream_t>(stream));
    if (dst_ != ATTN_OK) return dst_;
  }
  // padding rows: +0.0, one pass; the attention writes every indexed row
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (attnfwd::launch_scatter(nullptr, out, indices, n_valid, n_rows, out_row_bytes, s) !=
      hipSuccess)
    return ATTN_ERR_HIP;
  if (!work) return ATTN_OK;
  const int max_q = max_seqlen < n_valid ? max_seqlen : n_valid;
  return launch(a, head_dim, true, max_q, nullptr, 0, s);
}

int64_t attn_bwd_workspace_bytes(int64_t total_q, int32_t num_heads_q) {
  if (total_q <= 0 || num_heads_q <= 0) return 0;
  return total_q * num_heads_q * 4;
}

attn_status_t attn_bwd_varlen(const void* q, const void* k, const void* v, const float* out,
                              const void* dout, const float* lse, const int32_t* cu_seqlens_q,
                              const int32_t* cu_seqlens_k, int32_t num_seqs, int32_t total_q,
                              int32_t total_k, int32_t num_heads_q, int32_t num_heads_k,
                              int32_t head_dim, int32_t max_seqlen_q, int32_t max_seqlen_k,
                              float scale, int32_t causal, float* dq, float* dk, float* dv,
                              void* workspace, int64_t workspace_bytes, void* stream) {
  if (num_seqs < 0 || total_q < 0 || total_k < 0 || max_seqlen_q < 0 || max_seqlen_k < 0)
    return ATTN_ERR_SHAPE;
  attn_status_t st = check_common(num_heads_q, num_heads_k, head_dim, scale);
  if (st != ATTN_OK) return st;
  if (head_dim != 32 && head_dim != 64 && head_dim != 128 && head_dim != 256) return ATTN_ERR_UNSUPPORTED;
  if (workspace_bytes < 0) return ATTN_ERR_SHAPE;
  if (num_seqs == 0 || num_heads_q == 0 || (total_q == 0 && total_k == 0)) return ATTN_OK;
  if ((total_q > 0 && max_seqlen_q == 0) || (total_k > 0 && max_seqlen_k == 0)) return ATTN_ERR_SHAPE;
  if (cu_seqlens_q == nullptr || cu_seqlens_k == nullptr) return ATTN_ERR_NULL;
  if (!aligned4(cu_seqlens_q) || !aligned4(cu_seqlens_k)) return ATTN_ERR_ALIGN;
  st = check_bwd_ptrs(q, k, v, out, dout, lse, dq, dk, dv, workspace);
  if (st != ATTN_OK) return st;
  AttnArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = const_cast<float*>(out);
  a.lse = const_cast<float*>(lse);
  a.cu_q = cu_seqlens_q;
  a.cu_k = cu_seqlens_k;
  a.q_ss = (int64_t)num_heads_q * head_dim;
  a.q_hs = head_dim;
  a.k_ss = (int64_t)num_heads_k * head_dim;
  a.k_hs = head_dim;
  a.v_ss = a.k_ss;
  a.v_hs = head_dim;
  a.o_ss = a.q_ss;
  a.o_hs = head_dim;
  a.lse_hs = total_q;
  a.nseq = num_seqs;
  a.hq = num_heads_q;
  a.hkv = num_heads_k;
  a.group = num_heads_q / num_heads_k;
  a.c = base2_factor(scale);
  a.causal = causal ? 1 : 0;
  if (!span_fits(total_q, a.q_ss) || !span_fits(total_k, a.k_ss)) return ATTN_ERR_SHAPE;
  st = run_debug({cu_check(cu_seqlens_q, num_seqs, total_q, max_seqlen_q),
                  cu_check(cu_seqlens_k, num_seqs, total_k, max_seqlen_k)},
                 static_cast<hipStream_t>(stream));
  if (st != ATTN_OK) return st;
  const int max_q = max_seqlen_q < total_q ? max_seqlen_q : total_q;
  const int max_k = max_seqlen_k < total_k ? max_seqlen_k : total_k;
  return launch_bwd(a, head_dim, true, max_q, max_k, total_q, dout, dq, dk, dv, workspace,
                    workspace_bytes, static_cast<hipStream_t>(stream));
}

attn_status_t attn_bwd_dense(const void* q, const void* k, const void* v, const float* out,
                             const void* dout, const float* lse, int32_t batch, int32_t seqlen_q,
                             int32_t seqlen_k, int32_t num_heads_q, int32_t num_heads_k,
                             int32_t head_dim, float scale, int32_t causal, float* dq, float* dk,
                             float* dv, void* workspace, int64_t workspace_bytes, void* stream) {
  if (batch < 0 || seqlen_q < 0 || seqlen_k < 0) return ATTN_ERR_SHAPE;
  attn_status_t st = check_common(num_heads_q, num_heads_k, head_dim, scale);
  if (st != ATTN_OK) return st;
  if (head_dim != 32 && head_dim != 64 && head_dim != 128 && head_dim != 256) return ATTN_ERR_UNSUPPORTED;
  if (workspace_bytes < 0) return ATTN_ERR_SHAPE;
  if (batch == 0 || num_heads_q == 0 || (seqlen_q == 0 && seqlen_k == 0)) return ATTN_OK;
  st = check_bwd_ptrs(q, k, v, out, dout, lse, dq, dk, dv, workspace);
  if (st != ATTN_OK) return st;
  AttnArgs a{};
  const int64_t d = head_dim;
  a.q_hs = d;
  a.q_ss = num_heads_q * d;
  a.q_bs = a.q_ss * seqlen_q;
  a.k_hs = d;
  a.k_ss = num_heads_k * d;
  a.k_bs = a.k_ss * seqlen_k;
  a.v_hs = d;
  a.v_ss = a.k_ss;
  a.v_bs = a.k_bs;
  a.o_hs = d;
  a.o_ss = a.q_ss;
  a.o_bs = a.q_bs;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = const_cast<float*>(out);
  a.lse = const_cast<float*>(lse);
  a.lse_hs = seqlen_q;
  a.lse_bs = (int64_t)num_heads_q * seqlen_q;
  a.nseq = batch;
  a.hq = num_heads_q;
  a.hkv = num_heads_k;
  a.group = num_heads_q / num_heads_k;
  a.sq = seqlen_q;
  a.sk = seqlen_k;
  a.c = base2_factor(scale);
  a.causal = causal ? 1 : 0;
  if (!span_fits(seqlen_q, a.q_ss) || !span_fits(seqlen_k, a.k_ss)) return ATTN_ERR_SHAPE;
  return launch_bwd(a, head_dim, false, seqlen_q, seqlen_k, (int64_t)batch * seqlen_q, dout, dq,
                    dk, dv, workspace, workspace_bytes, static_cast<hipStream_t>(stream));
}

int64_t attn_fwd_paged_workspace_bytes(int32_t num_seqs, int32_t max_seqlen_q,
                                       int32_t max_seqlen_k, int32_t num_heads_q,
                                       int32_t num_heads_k, int32_t head_dim) {
  if (num_seqs <= 0 || max_seqlen_q <= 0 || max_seqlen_k <= 0 || num_heads_q <= 0 ||
      num_heads_k <= 0 || num_heads_q % num_heads_k != 0 || !head_dim_ok(head_dim))
    return 0;
  const PagedPlan p = plan_paged(num_seqs, max_seqlen_q, max_seqlen_k, num_heads_q / num_heads_k,
                                 num_heads_k);
  return paged_workspace_bytes(p, num_seqs, num_heads_k, head_dim);
}

attn_status_t attn_fwd_paged(const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* cu_seqlens_q, const int32_t* seqlens_k,
                             const int32_t* block_table, int32_t num_seqs, int32_t total_q,
                             int32_t num_pages, int32_t page_size, int32_t max_pages_per_seq,
                             int32_t num_heads_q, int32_t num_heads_k, int32_t head_dim,
                             int32_t max_seqlen_q, int32_t max_seqlen_k, float scale,
                             int32_t causal, float* out, float* lse, void* workspace,
                             int64_t workspace_bytes, void* stream) {
  return paged_impl(q, k_cache, v_cache, cu_seqlens_q, seqlens_k, block_table, num_seqs, total_q,
                    num_pages, page_size, max_pages_per_seq, num_heads_q, num_heads_k, head_dim,
                    max_seqlen_q, max_seqlen_k, scale, causal, out, lse, workspace,
                    workspace_bytes, false, 1.f, 1.f, stream);
}

attn_status_t attn_fwd_paged_fp8kv(const void* q, const void* k_cache, const void* v_cache,
                                   const int32_t* cu_seqlens_q, const int32_t* seqlens_k,
                                   const int32_t* block_table, int32_t num_seqs, int32_t total_q,
                                   int32_t num_pages, int32_t page_size, int32_t max_pages_per_seq,
                                   int32_t num_heads_q, int32_t num_heads_k, int32_t head_dim,
                                   int32_t max_seqlen_q, int32_t max_seqlen_k, float scale,
                                   float k_scale, float v_scale, int32_t causal, float* out,
                                   float* lse, void* workspace, int64_t workspace_bytes,
                                   void* stream) {
  return paged_impl(q, k_cache, v_cache, cu_seqlens_q, seqlens_k, block_table, num_seqs, total_q,
                    num_pages, page_size, max_pages_per_seq, num_heads_q, num_heads_k, head_dim,
                    max_seqlen_q, max_seqlen_k, scale, causal, out, lse, workspace,
                    workspace_bytes, true, k_scale, v_scale, stream);
}

attn_status_t attn_fwd_paged_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                     const int32_t* cu_seqlens_q, const int32_t* seqlens_k,
                                     const int32_t* block_table, int32_t num_seqs,
                                     int32_t total_q, int32_t num_pages, int32_t page_size,
                                     int32_t max_pages_per_seq, int32_t num_heads_q,
                                     int32_t num_heads_k, int32_t head_dim, int32_t max_seqlen_q,
                                     int32_t max_seqlen_k, float scale, int32_t causal,
                                     float* out, float* lse, void* stream) {
  return paged_impl(q, k_cache, v_cache, cu_seqlens_q, seqlens_k, block_table, num_seqs, total_q,
                    num_pages, page_size, max_pages_per_seq, num_heads_q, num_heads_k, head_dim,
                    max_seqlen_q, max_seqlen_k, scale, causal, out, lse, nullptr, 0, false, 1.f,
                    1.f, stream, true);
}

attn_status_t attn_mask_to_varlen(const void* mask, int32_t batch, int32_t seqlen,
                                  int32_t* indices, int32_t* cu_seqlens, int32_t* stats,
                                  void* stream) {
  if (batch < 0 || seqlen < 0) return ATTN_ERR_SHAPE;
  if ((int64_t)batch * seqlen >= (1LL << 31)) return ATTN_ERR_SHAPE;
  if (cu_seqlens == nullptr || stats == nullptr) return ATTN_ERR_NULL;
  if (batch > 0 && seqlen > 0 && (mask == nullptr || indices == nullptr)) return ATTN_ERR_NULL;
  if (!aligned4(cu_seqlens) || !aligned4(stats) || (indices && !aligned4(indices)))
    return ATTN_ERR_ALIGN;
  const hipError_t e = attnfwd::launch_mask_to_varlen(
      static_cast<const uint8_t*>(mask), batch, seqlen, indices, cu_seqlens, stats,
      static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

attn_status_t attn_fwd_fp8_varlen(const void* q, const void* k, const void* v,
                                  const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                  int32_t num_seqs, int32_t total_q, int32_t total_k,
                                  int32_t num_heads_q, int32_t num_heads_k, int32_t head_dim,
                                  int32_t max_seqlen, float scale, float q_scale, float k_scale,
                                  float v_scale, int32_t causal, float* out, float* lse,
                                  void* stream) {
  if (num_seqs < 0 || total_q < 0 || total_k < 0 || max_seqlen < 0) return ATTN_ERR_SHAPE;
  attn_status_t st = check_fp8(num_heads_q, num_heads_k, head_dim, scale, q_scale, k_scale, v_scale);
  if (st != ATTN_OK) return st;
  if (num_seqs == 0 || total_q == 0 || num_heads_q == 0) return ATTN_OK;
  if (max_seqlen == 0) return ATTN_ERR_SHAPE;
  if (q == nullptr || out == nullptr || cu_seqlens_q == nullptr || cu_seqlens_k == nullptr)
    return ATTN_ERR_NULL;
  if (total_k > 0 && (k == nullptr || v == nullptr)) return ATTN_ERR_NULL;
  if (!aligned16(q) || !aligned16(out) || (total_k > 0 && (!aligned16(k) || !aligned16(v))))
    return ATTN_ERR_ALIGN;
  if (!aligned4(cu_seqlens_q) || !aligned4(cu_seqlens_k) || (lse && !aligned4(lse)))
    return ATTN_ERR_ALIGN;
  AttnArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = out;
  a.lse = lse;
  a.cu_q = cu_seqlens_q;
  a.cu_k = cu_seqlens_k;
  a.q_ss = (int64_t)num_heads_q * head_dim;  // bytes
  a.q_hs = head_dim;
  a.k_ss = (int64_t)num_heads_k * head_dim;
  a.k_hs = head_dim;
  a.v_ss = a.k_ss;
  a.v_hs = head_dim;
  a.o_ss = (int64_t)num_heads_q * head_dim;  // fp32 elements
  a.o_hs = head_dim;
  a.lse_hs = total_q;
  a.nseq = num_seqs;
  a.hq = num_heads_q;
  a.hkv = num_heads_k;
  a.group = num_heads_q / num_heads_k;
  a.causal = causal ? 1 : 0;
  if ((int64_t)total_q * a.q_ss >= (1LL << 32) || (int64_t)total_k * a.k_ss >= (1LL << 32))
    return ATTN_ERR_SHAPE;
  st = run_debug({cu_check(cu_seqlens_q, num_seqs, total_q, max_seqlen),
                  cu_check(cu_seqlens_k, num_seqs, total_k, -1)},
                 static_cast<hipStream_t>(stream));
  if (st != ATTN_OK) return st;
  const int max_q = max_seqlen < total_q ? max_seqlen : total_q;
  return launch_fp8(a, head_dim, true, max_q, scale, q_scale, k_scale, v_scale,
                    static_cast<hipStream_t>(stream));
}

attn_status_t attn_fwd_fp8_dense(const void* q, const void* k, const void* v, int32_t batch,
                                 int32_t seqlen_q, int32_t seqlen_k, int32_t num_heads_q,
                                 int32_t num_heads_k, int32_t head_dim, float scale,
                                 float q_scale, float k_scale, float v_scale, int32_t causal,
                                 float* out, float* lse, void* stream) {
  if (batch < 0 || seqlen_q < 0 || seqlen_k < 0) return ATTN_ERR_SHAPE;
  attn_status_t st = check_fp8(num_heads_q, num_heads_k, head_dim, scale, q_scale, k_scale, v_scale);
  if (st != ATTN_OK) return st;
  if (batch == 0 || seqlen_q == 0 || num_heads_q == 0) return ATTN_OK;
  if (q == nullptr || out == nullptr) return ATTN_ERR_NULL;
  if (seqlen_k > 0 && (k == nullptr || v == nullptr)) return ATTN_ERR_NULL;
  if (!aligned16(q) || !aligned16(out) || (seqlen_k > 0 && (!aligned16(k) || !aligned16(v))))
    return ATTN_ERR_ALIGN;
  if (lse && !aligned4(lse)) return ATTN_ERR_ALIGN;
  AttnArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = out;
  a.lse = lse;
  a.q_hs = head_dim;
  a.q_ss = (int64_t)num_heads_q * head_dim;
  a.k_hs = head_dim;
  a.k_ss = (int64_t)num_heads_k * head_dim;
  a.v_hs = head_dim;
  a.v_ss = a.k_ss;
  a.o_hs = head_dim;
  a.o_ss = (int64_t)num_heads_q * head_dim;
  a.o_bs = a.o_ss * seqlen_q;
  a.lse_hs = seqlen_q;
  a.lse_bs = (int64_t)num_heads_q * seqlen_q;
  a.nseq = batch;
  a.hq = num_heads_q;
  a.hkv = num_heads_k;
  a.group = num_heads_q / num_heads_k;
  a.sq = seqlen_q;
  a.sk = seqlen_k;
  a.causal = causal ? 1 : 0;
  if ((int64_t)seqlen_q * a.q_ss >= (1LL << 32) || (int64_t)seqlen_k * a.k_ss >= (1LL << 32))
    return ATTN_ERR_SHAPE;
  return launch_fp8(a, head_dim, false, seqlen_q, scale, q_scale, k_scale, v_scale,
                    static_cast<hipStream_t>(stream));
}

attn_status_t attn_unpad_gather(const void* const* src, void* const* dst, int32_t n_tensors,
                                const int32_t* indices, int32_t n_valid, int32_t n_rows_src,
                                int64_t row_bytes, void* stream) {
  if (n_tensors < 1 || n_tensors > 3) return ATTN_ERR_SHAPE;
  if (n_valid < 0 || n_rows_src < 0 || row_bytes <= 0) return ATTN_ERR_SHAPE;
  if (row_bytes % 16 != 0) return ATTN_ERR_ALIGN;
  if (n_valid == 0) return ATTN_OK;
  if (src == nullptr || dst == nullptr || indices == nullptr) return ATTN_ERR_NULL;
  for (int t = 0; t < n_tensors; ++t) {
    if (dst[t] == nullptr || (n_rows_src > 0 && src[t] == nullptr)) return ATTN_ERR_NULL;
    if (!aligned16(dst[t]) || !aligned16(src[t])) return ATTN_ERR_ALIGN;
  }
  if (!aligned4(indices)) return ATTN_ERR_ALIGN;
  if ((int64_t)n_valid * (row_bytes / 16) >= (1LL << 32)) return ATTN_ERR_SHAPE;
  hipError_t e = attnfwd::launch_gather(src, dst, n_tensors, indices, n_valid, n_rows_src,
                                        row_bytes, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

attn_status_t attn_pad_scatter(const void* src, void* dst, const int32_t* indices, int32_t n_valid,
                               int32_t n_rows_total, int64_t row_bytes, void* stream) {
  if (n_valid < 0 || n_rows_total < 0 || row_bytes <= 0) return ATTN_ERR_SHAPE;
  if (row_bytes % 16 != 0) return ATTN_ERR_ALIGN;
  if (n_valid > n_rows_total) return ATTN_ERR_SHAPE;
  if (n_rows_total == 0) return ATTN_OK;
  if (dst == nullptr) return ATTN_ERR_NULL;
  if (n_valid > 0 && (src == nullptr || indices == nullptr)) return ATTN_ERR_NULL;
  if (!aligned16(dst) || (n_valid > 0 && (!aligned16(src) || !aligned4(indices))))
    return ATTN_ERR_ALIGN;
  if ((int64_t)n_rows_total * (row_bytes / 16) >= (1LL << 31)) return ATTN_ERR_SHAPE;
  if (n_valid > 0) {
    const attn_status_t dst_ =
        run_debug({idx_check(indices, n_valid, -1)}, static_cast<hipStream_t>(stream));
    if (dst_ != ATTN_OK) return dst_;
  }
  hipError_t e = attnfwd::launch_scatter(src, dst, indices, n_valid, n_rows_total, row_bytes,
                                         static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

const char* attn_status_str(attn_status_t s) {
  switch (s) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "a required pointer is NULL";
    case ATTN_ERR_SHAPE: return "invalid or inconsistent sizes";
    case ATTN_ERR_SCRATCH: return "the call needs more scratch memory than the library's static buffer holds";
    case ATTN_ERR_UNSUPPORTED: return "unsupported argument (head_dim must be 32/64/128/256; scale finite; or a policy/order this launch cannot use)";
    case ATTN_ERR_ALIGN: return "pointer, stride or row size not 16-byte aligned";
    case ATTN_ERR_HIP: return "HIP runtime rejected the launch";
    default: return "unknown status";
  }
}

int32_t attn_abi_version(void) { return ATTN_FWD_ABI_VERSION; }

}  // extern "C"
