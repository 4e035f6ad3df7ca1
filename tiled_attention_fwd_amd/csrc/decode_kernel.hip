// Attention of new queries over a paged KV cache (decode / speculative /
// chunked prefill), gfx950.
//
// Page "why FA is 2x on A100 but 1.5x on Ascend 910", section 5: inference
// keeps the KV cache in pages handed out by a page table (PagedAttention) and
// is limited by moving K and V, not by arithmetic.  Key j of sequence s is row
// j % page_size of page block_table[s][j / page_size]; the new queries of s
// (rows cu_q[s] .. cu_q[s+1] of q) attend to its seqlens_k[s] keys, causal
// with bottom-right alignment.  The attention is the one of page "Intro to
// FlashAttention on Ascend CANN" (online softmax over key tiles, "the first
// pitfall"), and key ranges split over workgroups are combined from their
// partial results and log-sum-exps, which that section's merge rule makes
// exact.
//
// Design (bound by HBM: K and V of every (sequence, KV head) are read once):
//  * The MFMA's 32 query columns hold (query, head-of-group) pairs of one KV
//    head: row r = qi * group + g.  A decode step of a GQA model (1 query, 8
//    heads per KV head) fills 8 columns and reads each K/V byte once for all
//    8 heads.  More rows than 32 use further row blocks.
//  * A workgroup owns (sequence, KV head, row block, key chunk); its waves take
//    the chunk's 32-key tiles round-robin, each streaming its own tiles by LDS
//    DMA into private double buffers (no workgroup barrier in the loop), with
//    the page lookup done per DMA instruction.  Rows past the sequence's
//    length or page read as zero through the buffer range check.
//  * At the end the waves merge (m, l, O) through LDS; the workgroup writes the
//    final output, or a normalised partial and its base-2 LSE when the key
//    range is split, and decode_merge_kernel combines the parts.

#include "decode_internal.h"
#include "attn_device.h"

#include <math.h>

#include <type_traits>

namespace attnfwd {
namespace {

constexpr int kTileKeys = 32;


// 32-row tiles, row-major with a 16-byte chunk swizzle.  DMA lanes are
// row-major (lane i of an instruction carries row i / CPR, so each quad of
// lanes reads one aligned 64-byte segment of a source row); the slot at
// position p of row r holds chunk p ^ swz(r).  K rows hold key key_of_row(r)
// (the accumulator order the P operand needs), V rows their own key.  The
// swizzles make the K row fragments and the V transposed fragments free of
// bank conflicts (at d=32 a row is one 64-byte segment: K rotates by (r / 4)
// mod 4 chunks, V needs none).
template <int D>
struct RowTile {
  static constexpr int CPR = D / 8;        // 16-byte chunks per row
  static constexpr int R = 64 / CPR;       // rows per DMA instruction
  static constexpr int PITCH = 2 * D;      // bytes per row
  static constexpr int BYTES = kTileKeys * PITCH;
  static_assert(D == 32 || D == 64 || D == 128 || D == 256, "tile layout defined for head_dim 32..256");
  static __device__ __forceinline__ int swz_k(int row) {
    return D >= 128 ? (row & 15) : (D == 64 ? ((row >> 1) & 7) : ((row >> 2) & 3));
  }
  static __device__ __forceinline__ int swz_v(int row) {
    return D >= 128 ? ((row & 3) << 2) : (D == 64 ? (((row >> 1) & 1) << 2) : 0);
  }
};

template <int D>
struct Frag32 {
  using L = RowTile<D>;
  static constexpr int NDB = D / 32;
  int rd_row;      // l32 * PITCH
  int rd_x;        // swz_k(l32)
  int hh;
  int tr_base;     // (8 hh + u) * PITCH + 16 cc + 8 (lane & 1)
  int tr_db[NDB];  // 64 * (db ^ (swz_v / 4)) per column block
  __device__ __forceinline__ void init(int lane) {
    const int l32 = lane & 31;
    hh = lane >> 5;
    rd_row = l32 * L::PITCH;
    rd_x = L::swz_k(l32);
    const int u = (lane & 15) >> 2;
    const int cc = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    tr_base = (8 * hh + u) * L::PITCH + 16 * cc + 8 * (lane & 1);
    const int xs = L::swz_v(u) >> 2;  // swz_v of row 16 tt + 8 hh + 4 hi + u depends on u only
#pragma unroll
    for (int db = 0; db < NDB; ++db) tr_db[db] = 64 * (db ^ xs);
  }
  // rows 0..31 (LDS order), dims 16 s .. 16 s + 15
  __device__ __forceinline__ bf16x8 row(const unsigned char* t, int s) const {
    return *reinterpret_cast<const bf16x8*>(t + rd_row + 16 * ((2 * s + hh) ^ rd_x));
  }
  // dims 32 db .. 32 db + 31 by natural rows 16 tt .. 16 tt + 15
  __device__ __forceinline__ bf16x8 trn(const unsigned char* t, int tt, int db) const {
    const unsigned char* p = t + tr_base + tr_db[db] + 16 * tt * L::PITCH;
    const uint2 lo = ds_read_tr16(reinterpret_cast<const uint16_t*>(p));
    const uint2 hi = ds_read_tr16(reinterpret_cast<const uint16_t*>(p + 4 * L::PITCH));
    return as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
  }
};

template <int D>
constexpr int tile32_bytes() { return RowTile<D>::BYTES; }

// E4M3 cache tiles: 32 rows of D bytes, row-major DMA lanes, and XOR chunk
// swizzles of row bits for the two reads below (16-byte K row reads, 8-byte
// transposed V reads of eight rows): K chunk (r ^ r/2) mod 16 / 8, (r ^ r/4)
// mod 4, (r/4 ^ r/8) mod 2 and V chunk (r ^ r/2) mod 8 / 8 / 4 (mod 4 at
// d=64), (r ^ r/4) mod 2 at head_dim 256 / 128 / 64 / 32.  A host model of
// the placement and reads finds them free of bank conflicts except the V reads
// at head_dim 256 (one of the two phase groupings, 2-way).  The V swizzle uses
// row bits 0..3 only, so it is a lane constant for both 16-row halves of a
// tile.  At head_dim 32 one DMA instruction carries all 32 rows (both 16-key
// groups, which may lie in different pages), so it is issued once per group
// with the other group's lanes off.  The fragments are dequantised to bf16 in
// registers (E4M3 values are exact in bf16), so the products stay bf16 MFMAs
// with exact operands.
template <int D>
struct RowTile8 {
  static constexpr int CPR = D / 16;   // 16-byte chunks per row
  static constexpr int R = 64 / CPR;   // rows per DMA instruction
  static constexpr int PITCH = D;
  static constexpr int BYTES = kTileKeys * PITCH;
  static __device__ __forceinline__ int swz_k(int r) {
    return D == 256 ? ((r ^ (r >> 1)) & 15)
                    : D == 128 ? ((r ^ (r >> 1)) & 7) : D == 64 ? ((r ^ (r >> 2)) & 3) : (((r >> 2) ^ (r >> 3)) & 1);
  }
  static __device__ __forceinline__ int swz_v(int r) {
    return D >= 128 ? ((r ^ (r >> 1)) & 7) : D == 64 ? ((r ^ (r >> 1)) & 3) : ((r ^ (r >> 2)) & 1);
  }
};

typedef int i32x2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(uint32_t lo, uint32_t hi) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// K: one 16-byte read per pair of score MFMAs.  Pair j covers dims 32 j ..
// 32 j + 31: lane half hh holds dims 32 j + 16 hh + 8 sub + e for MFMA
// (j, sub) (Q uses the same assignment, which is all the MFMA needs).
// V: ds_read_b64_tr_b8 gives a lane 8 consecutive keys of one dim.
template <int D>
struct Frag32F8 {
  using L = RowTile8<D>;
  static constexpr int NDB = D / 32;
  int rd_row, rd_x, hh, tr_base;
  __device__ __forceinline__ void init(int lane) {
    const int l32 = lane & 31;
    hh = lane >> 5;
    rd_row = l32 * L::PITCH;
    rd_x = L::swz_k(l32);
    const int vg = (lane >> 4) & 1, vi = lane & 15;
    // natural row 16 tt + 8 hh + vi / 2: swz_v uses row bits 0..3 only
    tr_base = (8 * hh + (vi >> 1)) * L::PITCH + 8 * (vi & 1) + 16 * vg;
    tr_x = L::swz_v(8 * hh + (vi >> 1));
    tr_vg = vg;
  }
  int tr_x, tr_vg;
  __device__ __forceinline__ void krow(const unsigned char* t, int j, bf16x8& a0, bf16x8& a1) const {
    const uint4 x = *reinterpret_cast<const uint4*>(t + rd_row + 16 * ((2 * j + hh) ^ rd_x));
    a0 = e4m3x8_to_bf16(x.x, x.y);
    a1 = e4m3x8_to_bf16(x.z, x.w);
  }
  __device__ __forceinline__ bf16x8 vtr(const unsigned char* t, int tt, int db) const {
    const int c = 2 * db + tr_vg;
    const unsigned char* p = t + tr_base - 16 * tr_vg + 16 * (c ^ tr_x) + 16 * tt * L::PITCH;
    const i32x2v x = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
        (__attribute__((address_space(3))) i32x2v*)(p));
    return e4m3x8_to_bf16((uint32_t)x[0], (uint32_t)x[1]);
  }
};

// Pages of one 32-key tile: its two aligned 16-key groups (the same page when
// page_size >= 32).  A group past the sequence, past the table row or naming a
// page outside the pool is dead: its loads get an empty buffer range, so its
// lanes read zeros and nothing is dereferenced.
struct TilePages {
  const unsigned char* kbase[2];
  const unsigned char* vbase[2];
  uint32_t bytes[2];
  int pstart[2];
};

// page[g] is the table entry of the tile's 16-key group g (-1: none).
template <int D, int ES>
__device__ __forceinline__ TilePages tile_pages(const DecodeArgs& a, const int page[2], int lk,
                                                int kvh, int t) {
  TilePages tp;
  const uint32_t row_bytes = (uint32_t)a.hkv * D * ES;
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const int key0 = t * kTileKeys + 16 * g;
    const int pidx = key0 / a.page_size;
    const int pg = page[g];
    const bool live = key0 < lk && pidx < a.max_pages && pg >= 0 && pg < a.num_pages;
    tp.pstart[g] = pidx * a.page_size;
    const int valid = min(a.page_size, lk - tp.pstart[g]);  // >= 1 when key0 < lk
    const int64_t off = ((int64_t)(live ? pg : 0) * a.page_size * a.hkv + kvh) * D * ES;
    tp.kbase[g] = reinterpret_cast<const unsigned char*>(a.k_cache) + off;
    tp.vbase[g] = reinterpret_cast<const unsigned char*>(a.v_cache) + off;
    tp.bytes[g] = live ? (uint32_t)(valid - 1) * row_bytes + D * ES : 0u;
  }
  return tp;
}

// Table entries of the 16-key groups of up to 32 of this wave's tiles, one
// per lane: lane i holds group i % 2 of tile j0 + i / 2 (-1 past the wave's
// tiles, the sequence or the table row).  One vector load replaces a
// dependent table read before every tile's DMA.
__device__ __forceinline__ int load_pages(const DecodeArgs& a, const int32_t* table_row, int lk,
                                          int first, int stride, int n_mine, int j0, int lane) {
  const int jj = j0 + (lane >> 1);
  const int key0 = (first + jj * stride) * kTileKeys + 16 * (lane & 1);
  const int pidx = key0 / a.page_size;
  int pg = -1;
  if (jj < n_mine && key0 < lk && pidx < a.max_pages) pg = table_row[pidx];
  return pg;
}

// DMA of keys 32 t .. 32 t + 31 of one (sequence, KV head) from the cache into
// a 32-row tile at LDS byte address `tile`.  Instruction q carries tile rows
// q R .. q R + R - 1, whose source keys (key_of_row of the row) lie in the
// aligned 16-key group (q R) / 16, hence in one page (page_size is a multiple
// of 16).
template <int D, int ES>
using TileOf = typename std::conditional<ES == 2, RowTile<D>, RowTile8<D>>::type;

// DMA instructions per 32-key tile and tensor (an instruction carrying both
// 16-key groups is issued once per group)
template <int D, int ES>
constexpr int dma_per_tile() {
  return TileOf<D, ES>::R > 16 ? 2 : kTileKeys / TileOf<D, ES>::R;
}

template <int D, int ES>
__device__ __forceinline__ void dma_tile(const TilePages& tp, bool is_v, int hkv, int t,
                                         uint32_t tile, int lane) {
  using L = TileOf<D, ES>;
  constexpr int R = L::R;
  constexpr int NQ = R > 16 ? 1 : kTileKeys / R;
  const int p = lane % L::CPR;
  const uint32_t row_bytes = (uint32_t)hkv * D * ES;
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int row = q * R + lane / L::CPR;
    const int key = t * kTileKeys + (is_v ? row : key_of_row(row));
    const int c = p ^ (is_v ? L::swz_v(row) : L::swz_k(row));
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(tile + q * 1024);
    if constexpr (R > 16) {
      // rows 0..15 and 16..31 (their keys too) are the tile's two 16-key groups
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        if ((row >> 4) == g) {
          const u32x4 desc = make_desc(is_v ? tp.vbase[g] : tp.kbase[g], tp.bytes[g]);
          dma16(desc, (uint32_t)(key - tp.pstart[g]) * row_bytes + (uint32_t)c * 16, m0);
        }
      }
    } else {
      const int g = (q * R) >> 4;
      const u32x4 desc = make_desc(is_v ? tp.vbase[g] : tp.kbase[g], tp.bytes[g]);
      dma16(desc, (uint32_t)(key - tp.pstart[g]) * row_bytes + (uint32_t)c * 16, m0);
    }
  }
}

template <int NI>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NI) : "memory");
}

// Waits until a wave's oldest tile has landed while `after` later tiles (each
// 2 NI loads: K and V) may stay in flight; only the counts a stage depth can
// reach are instantiated.
template <int NI, int NBUF>
__device__ __forceinline__ void wait_tile(int after) {
  if constexpr (NBUF >= 4) {
    if (after >= 3) { wait_vm<6 * NI>(); return; }
  }
  if constexpr (NBUF >= 3) {
    if (after == 2) { wait_vm<4 * NI>(); return; }
  }
  if (after >= 1) { wait_vm<2 * NI>(); return; }
  wait_vm<0>();
}

constexpr float kLazyRescale = 8.0f;

// Two workgroups per CU when one takes at most half of the LDS and four waves:
// then each may use 256 registers, so two waves share a SIMD.
template <int D, int WAVES, int NBUF, int ES>
constexpr int decode_min_waves() {
  constexpr int tb = 32 * D * ES;  // bytes of a 32-key tile of K (or V)
  constexpr int lds_w = WAVES * NBUF * 2 * tb;
  constexpr int lds_m = WAVES * (32 * D + 64) * 4;
  return (WAVES <= 4 && D <= 128 && (lds_w > lds_m ? lds_w : lds_m) <= 80 * 1024) ? 2 : 1;
}

template <int D, int WAVES, int NBUF, int ES>
__global__ __launch_bounds__(WAVES * 64, (decode_min_waves<D, WAVES, NBUF, ES>())) void attn_decode_kernel(const DecodeArgs a) {
  constexpr int NDS = D / 16, NDB = D / 32;
  using L = TileOf<D, ES>;
  constexpr int TB = L::BYTES;
  constexpr int NI = dma_per_tile<D, ES>();         // DMA instructions per tile per tensor
  constexpr int WAVE_LDS = NBUF * 2 * TB;           // NBUF stages of K and V
  constexpr int MERGE_LDS = WAVES * (32 * D + 64) * 4;
  constexpr int LDS = WAVES * WAVE_LDS > MERGE_LDS ? WAVES * WAVE_LDS : MERGE_LDS;
  static_assert(NBUF >= 2 && NBUF <= 4, "stage count");
  static_assert(2 * (NBUF - 1) * NI <= 63, "vmcnt range");
  __shared__ __attribute__((aligned(16))) unsigned char lds[LDS];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  // Grid order: KV head fastest (order 1: the workgroups that read the same
  // cache rows, which interleave the heads, run together), or key part fastest
  // (order 0).
  int x = blockIdx.x;
  int part, rb, kvh, seq;
  if (a.order == 1) {
    kvh = x % a.hkv;
    x /= a.hkv;
    rb = x % a.n_rb;
    x /= a.n_rb;
    part = x % a.n_split;
    seq = x / a.n_split;
  } else {
    part = x % a.n_split;
    x /= a.n_split;
    rb = x % a.n_rb;
    x /= a.n_rb;
    kvh = x % a.hkv;
    seq = x / a.hkv;
  }

  const DecodeRange dr = decode_range(a, seq, rb);
  if (dr.rows <= 0) return;
  const int parts = decode_parts(a, dr.n_kt);
  if (part >= parts) return;
  const int t_begin = part * a.chunk_tiles;
  const int t_end = a.n_split > 1 ? min(dr.n_kt, t_begin + a.chunk_tiles) : dr.n_kt;

  // this lane's column: row r of the block -> (query, head)
  const int r = rb * 32 + l32;
  const bool col_ok = r < dr.rows;
  const int qi = col_ok ? r / a.group : 0;
  const int hq = kvh * a.group + (col_ok ? r % a.group : 0);
  const int lim = !col_ok ? -1 : (a.causal ? min(dr.lk - 1, qi + dr.lk - dr.lq) : dr.lk - 1);
  // the smallest limit over the wave's valid columns: tiles whose keys all lie
  // at or below it need no mask (other columns are never stored)
  int lim_min = col_ok ? lim : 0x7fffffff;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) lim_min = min(lim_min, __shfl_xor(lim_min, o));
  lim_min = __builtin_amdgcn_readfirstlane(lim_min);

  // Q as the B operand.  bf16 cache: MFMA s takes dims 16 s + 8 hh + e; E4M3
  // cache: MFMA 2 j + sub takes dims 32 j + 16 hh + 8 sub + e (the order of
  // the dequantised K fragments).
  bf16x8 qf[NDS];
  {
    const uint16_t* qp = a.q + ((int64_t)(dr.q0 + qi) * a.hq + hq) * D;
#pragma unroll
    for (int s = 0; s < NDS; ++s) {
      const int dim0 = ES == 2 ? 16 * s + 8 * hh : 32 * (s >> 1) + 16 * hh + 8 * (s & 1);
      qf[s] = col_ok ? as_bf16x8(ld16(qp + dim0)) : bf16x8{};
    }
  }

  const int32_t* table_row = a.block_table + (int64_t)seq * a.max_pages;
  const uint32_t my_lds = lds_addr(lds) + wave * WAVE_LDS;
  const unsigned char* my_tiles = lds + wave * WAVE_LDS;
  typename std::conditional<ES == 2, Frag32<D>, Frag32F8<D>>::type fr;
  fr.init(lane);

  float m = -INFINITY, l = 0.f;
  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};

  // this wave's tiles: t_begin + wave + WAVES * j, j < n_mine; NBUF - 1 in flight
  const int first = t_begin + wave;
  const int n_mine = first < t_end ? (t_end - first + WAVES - 1) / WAVES : 0;
  int pagevec = load_pages(a, table_row, dr.lk, first, WAVES, n_mine, 0, lane);

  // issues tile j of this wave into buffer buf; tiles are issued in order, so
  // the page batch is reloaded when j crosses a multiple of 32 (a wave with
  // more than 32 tiles pays one drained load per 32 tiles)
  auto issue = [&](int j, int buf) {
    if (j > 0 && (j & 31) == 0)
      pagevec = load_pages(a, table_row, dr.lk, first, WAVES, n_mine, j, lane);
    const int t = first + j * WAVES;
    const int sel = 2 * (j & 31);
    const int page[2] = {__builtin_amdgcn_readlane(pagevec, sel),
                         __builtin_amdgcn_readlane(pagevec, sel + 1)};
    const uint32_t b = my_lds + buf * 2 * TB;
    const TilePages tp = tile_pages<D, ES>(a, page, dr.lk, kvh, t);
    dma_tile<D, ES>(tp, false, a.hkv, t, b, lane);
    dma_tile<D, ES>(tp, true, a.hkv, t, b + TB, lane);
  };

  // Every stage holds a tile in flight: a tile's K and V fragments are copied
  // to registers as soon as it lands, which frees its stage for the tile
  // NBUF ahead before any of the math runs.
#pragma unroll
  for (int j = 0; j < NBUF; ++j)
    if (j < n_mine) issue(j, j);
  for (int j = 0; j < n_mine; ++j) {
    const int t = first + j * WAVES;
    const int buf = j % NBUF;
    // tiles issued after tile j that may stay in flight
    const int after = min(NBUF - 1, n_mine - 1 - j);
    wait_tile<NI, NBUF>(after);
    const unsigned char* kt = my_tiles + buf * 2 * TB;
    const unsigned char* vt = kt + TB;
    bf16x8 kfr[NDS], vfr[2][NDB];
    if constexpr (ES == 2) {
#pragma unroll
      for (int s = 0; s < NDS; ++s) kfr[s] = fr.row(kt, s);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int db = 0; db < NDB; ++db) vfr[tt][db] = fr.trn(vt, tt, db);
    } else {
#pragma unroll
      for (int j2 = 0; j2 < NDS / 2; ++j2) fr.krow(kt, j2, kfr[2 * j2], kfr[2 * j2 + 1]);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int db = 0; db < NDB; ++db) vfr[tt][db] = fr.vtr(vt, tt, db);
    }
    if (j + NBUF < n_mine) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the reads of this stage are done
      issue(j + NBUF, buf);
    }
    f32x16 st = f32x16{};
#pragma unroll
    for (int s = 0; s < NDS; ++s)
      st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfr[s], qf[s], st, 0, 0, 0);
    // register e holds key 32 t + 16 (e / 8) + 8 hh + e % 8 for this column
    // scores in base-2 units first: c carries the scale's sign here
#pragma unroll
    for (int e = 0; e < 16; ++e) st[e] *= a.c;
    const int kbase = t * kTileKeys + hh * 8;
    if (t * kTileKeys + kTileKeys - 1 > lim_min) {
      keep_branch();
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (kbase + ((e >> 3) << 4) + (e & 7) > lim) st[e] = -INFINITY;
    }
    float mt = -INFINITY;
#pragma unroll
    for (int e = 0; e < 16; ++e) mt = fmaxf(mt, st[e]);
    mt = half_max(mt);
    // lazy reference maximum: m (and O, l) move only when a column's maximum
    // passes it by more than 2^8, so the bf16 probabilities stay <= 2^8
    const bool grow = mt > m + kLazyRescale;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float m_new = grow ? mt : m;
      const float alpha = grow ? __builtin_amdgcn_exp2f(m - m_new) : 1.f;  // 0 while m = -inf
      m = m_new;
      l *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[db][e] *= alpha;
    }
    const float mu = m == -INFINITY ? 0.f : m;
    float rs = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      st[e] = __builtin_amdgcn_exp2f(st[e] - mu);
      rs += st[e];
    }
    l += rs;
    bf16x8 pf[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      uint4 w;
      w.x = pack_bf16x2(st[8 * tt + 0], st[8 * tt + 1]);
      w.y = pack_bf16x2(st[8 * tt + 2], st[8 * tt + 3]);
      w.z = pack_bf16x2(st[8 * tt + 4], st[8 * tt + 5]);
      w.w = pack_bf16x2(st[8 * tt + 6], st[8 * tt + 7]);
      pf[tt] = as_bf16x8(w);
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vfr[tt][db], pf[tt], oacc[db], 0, 0, 0);
  }
  l = half_sum(l);

  // ---- merge the waves through LDS (the tile buffers are free after the barrier)
  __syncthreads();
  float* mo = reinterpret_cast<float*>(lds);  // [WAVES][32][D] then m, l [WAVES][32] each
  float* mm = mo + WAVES * 32 * D;
  float* ml = mm + WAVES * 32;
  {
    float* op = mo + (wave * 32 + l32) * D + hh * 4;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<float4*>(op + db * 32 + 8 * g) =
            make_float4(oacc[db][4 * g], oacc[db][4 * g + 1], oacc[db][4 * g + 2], oacc[db][4 * g + 3]);
    if (hh == 0) {
      mm[wave * 32 + l32] = m;
      ml[wave * 32 + l32] = l;
    }
  }
  __syncthreads();
  constexpr int CH = D / 4;  // float4 chunks per row
  for (int i = tid; i < 32 * CH; i += WAVES * 64) {
    const int col = i / CH, ch = i - col * CH;
    const int rr = rb * 32 + col;
    if (rr >= dr.rows) continue;
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) mx = fmaxf(mx, mm[w * 32 + col]);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    float lsum = 0.f;
    if (mx != -INFINITY) {
#pragma unroll
      for (int w = 0; w < WAVES; ++w) {
        const float f = __builtin_amdgcn_exp2f(mm[w * 32 + col] - mx);
        const float4 v = *reinterpret_cast<const float4*>(mo + (w * 32 + col) * D + 4 * ch);
        acc.x += f * v.x;
        acc.y += f * v.y;
        acc.z += f * v.z;
        acc.w += f * v.w;
        lsum += f * ml[w * 32 + col];
      }
    }
    // a split part stays normalised by its own sum; the v factor is applied once
    const float inv = lsum > 0.f ? (a.n_split > 1 ? 1.f : a.o_mul) / lsum : 0.f;
    acc.x *= inv;
    acc.y *= inv;
    acc.z *= inv;
    acc.w *= inv;
    const float lse2 = lsum > 0.f ? mx + __log2f(lsum) : -INFINITY;
    const int cq = rr / a.group;
    const int ch_q = kvh * a.group + rr % a.group;
    if (a.n_split > 1) {
      const int64_t pr = (((int64_t)seq * a.hkv + kvh) * a.n_rb + rb) * a.n_split + part;
      *reinterpret_cast<float4*>(a.part_o + (pr * 32 + col) * D + 4 * ch) = acc;
      if (ch == 0) a.part_lse[pr * 32 + col] = lse2;
    } else {
      *reinterpret_cast<float4*>(a.o + ((int64_t)(dr.q0 + cq) * a.hq + ch_q) * D + 4 * ch) = acc;
      if (ch == 0 && a.lse != nullptr)
        a.lse[(int64_t)ch_q * a.tq + dr.q0 + cq] = lse2 == -INFINITY ? -INFINITY : lse2 * kLn2;
    }
  }
}

// Combines the parts of split key ranges: O = sum_p 2^(L_p - L) O_p with
// L = log2 sum_p 2^(L_p).  One workgroup per (sequence, KV head, row block):
// 8 threads per row, D / 8 outputs each.
template <int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(const DecodeArgs a) {
  int x = blockIdx.x;
  const int rb = x % a.n_rb;
  x /= a.n_rb;
  const int kvh = x % a.hkv;
  const int seq = x / a.hkv;
  const DecodeRange dr = decode_range(a, seq, rb);
  const int col = threadIdx.x >> 3, sub = threadIdx.x & 7;
  const int rr = rb * 32 + col;
  if (dr.rows <= 0 || rr >= dr.rows) return;
  const int parts = decode_parts(a, dr.n_kt);
  const int64_t pr0 = (((int64_t)seq * a.hkv + kvh) * a.n_rb + rb) * a.n_split;
  float mx = -INFINITY;
  for (int p = 0; p < parts; ++p) mx = fmaxf(mx, a.part_lse[(pr0 + p) * 32 + col]);
  constexpr int PER = D / 8;
  float acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.f;
  float s = 0.f;
  if (mx != -INFINITY) {
    for (int p = 0; p < parts; ++p) {
      const float f = __builtin_amdgcn_exp2f(a.part_lse[(pr0 + p) * 32 + col] - mx);
      s += f;
      const float* src = a.part_o + ((pr0 + p) * 32 + col) * D + sub * 4;
#pragma unroll
      for (int i = 0; i < PER / 4; ++i) {
        const float4 v = *reinterpret_cast<const float4*>(src + 32 * i);
        acc[4 * i] += f * v.x;
        acc[4 * i + 1] += f * v.y;
        acc[4 * i + 2] += f * v.z;
        acc[4 * i + 3] += f * v.w;
      }
    }
  }
  const float inv = s > 0.f ? a.o_mul / s : 0.f;
  const int cq = rr / a.group;
  const int hq = kvh * a.group + rr % a.group;
  float* dst = a.o + ((int64_t)(dr.q0 + cq) * a.hq + hq) * D + sub * 4;
#pragma unroll
  for (int i = 0; i < PER / 4; ++i)
    *reinterpret_cast<float4*>(dst + 32 * i) =
        make_float4(acc[4 * i] * inv, acc[4 * i + 1] * inv, acc[4 * i + 2] * inv, acc[4 * i + 3] * inv);
  if (sub == 0 && a.lse != nullptr)
    a.lse[(int64_t)hq * a.tq + dr.q0 + cq] = s > 0.f ? (mx + __log2f(s)) * kLn2 : -INFINITY;
}

// Waves per workgroup and LDS stages per wave.  One workgroup fills most of a
// CU's LDS, so the product of the two is bounded by the tile size; the
// variants trade waves (latency hiding of the softmax/MFMA work) for stages
// (tiles in flight per wave).  d=128 (16 KiB per stage): 0 = 4 waves x 2
// stages, 1 = 3 x 3, 2 = 5 x 2; d=64 (8 KiB per stage) and d=32 (4 KiB):
// 0 = 4 x 4, 1 = 8 x 2, 2 = 5 x 4, 3 = 4 x 2 (two workgroups per CU).
template <int D, int W, int NB, int ES>
hipError_t launch_v(const DecodeArgs& a, int64_t grid, hipStream_t stream) {
  hipLaunchKernelGGL((attn_decode_kernel<D, W, NB, ES>), dim3((unsigned)grid), dim3(W * 64), 0,
                     stream, a);
  return hipSuccess;
}

template <int D>
hipError_t launch_d(const DecodeArgs& a, int variant, hipStream_t stream) {
  const int64_t grid = (int64_t)a.nseq * a.hkv * a.n_rb * a.n_split;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (grid == 0) return hipSuccess;
  // Defaults (variant < 0) from measured sweeps: more waves beat more stages
  // for bf16 caches (d=128 decode: 4x2 3.8, 3x3 3.6, 5x2 4.5 TB/s; d=64: 4x4
  // 3.4, 8x2 4.5, 5x4 4.2 TB/s).  E4M3 caches halve the stage size.
  if constexpr (D == 256) {
    // one wave per SIMD (each can hold a landed tile's fragments in
    // registers); a 32-key stage of K and V is 32 KiB (bf16) or 16 KiB (E4M3),
    // so two or four waves of two stages fill the LDS
    if (a.kv_fp8) launch_v<D, 4, 2, 1>(a, grid, stream);
    else launch_v<D, 2, 2, 2>(a, grid, stream);
  } else if constexpr (D == 32) {
    if (a.kv_fp8) launch_v<D, 8, 4, 1>(a, grid, stream);
    else if (variant == 0) launch_v<D, 4, 4, 2>(a, grid, stream);
    else if (variant == 2) launch_v<D, 5, 4, 2>(a, grid, stream);
    else launch_v<D, 8, 2, 2>(a, grid, stream);
  } else if (a.kv_fp8) {
    // E4M3 caches, d=128 decode b32 GQA-8 (cold): 4x4 195, 8x2 173, 5x4 184 us
    if constexpr (D == 128) {
      if (variant == 0) launch_v<D, 4, 4, 1>(a, grid, stream);
      else if (variant == 2) launch_v<D, 5, 4, 1>(a, grid, stream);
      else launch_v<D, 8, 2, 1>(a, grid, stream);
    } else {
      if (variant == 0) launch_v<D, 4, 4, 1>(a, grid, stream);
      else if (variant == 2) launch_v<D, 5, 4, 1>(a, grid, stream);
      else launch_v<D, 8, 4, 1>(a, grid, stream);
    }
  } else if constexpr (D == 128) {
    if (variant == 0) launch_v<D, 4, 2, 2>(a, grid, stream);
    else if (variant == 1) launch_v<D, 3, 3, 2>(a, grid, stream);
    else launch_v<D, 5, 2, 2>(a, grid, stream);
  } else {
    // A grid of at least two workgroups per CU with no split parts (many
    // short sequences): four waves of two stages take 64 KiB of LDS, so two
    // workgroups share a CU and one's start and merge overlap the other's
    // streaming (128 sequences x 32 heads, 1-2k keys, d=64, cold: 347 -> 325
    // us; 2 x 4 and 4 x 3 stages measured 377 and 422).  A split plan aims
    // at one workgroup per CU, which the eight-wave layout fills.
    const bool many = a.n_split == 1 && grid >= 512;
    if (variant == 0) launch_v<D, 4, 4, 2>(a, grid, stream);
    else if (variant == 2) launch_v<D, 5, 4, 2>(a, grid, stream);
    else if (variant == 3 || (variant < 0 && many && D == 64)) launch_v<D, 4, 2, 2>(a, grid, stream);
    else launch_v<D, 8, 2, 2>(a, grid, stream);
  }
  if (a.n_split > 1) {
    const int64_t gm = (int64_t)a.nseq * a.hkv * a.n_rb;
    hipLaunchKernelGGL((decode_merge_kernel<D>), dim3((unsigned)gm), dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int head_dim, int variant, hipStream_t stream) {
  switch (head_dim) {
    case 32: return launch_d<32>(a, variant, stream);
    case 64: return launch_d<64>(a, variant, stream);
    case 128: return launch_d<128>(a, variant, stream);
    case 256: return launch_d<256>(a, variant, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace attnfwd
