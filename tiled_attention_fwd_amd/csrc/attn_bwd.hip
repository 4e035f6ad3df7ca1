// FlashAttention backward for gfx950 (MI355X): gradients by recomputation.
//
// Page "Intro to FlashAttention on Ascend CANN", section on the second pitfall
// (backward propagation): the score matrix is not kept; the backward pass
// recomputes it tile by tile from Q, K and the forward's per-row log-sum-exp.
// With P = exp(scale * Q K^T - LSE) (masked entries 0) and the gradient dO of
// the output, the chain rule gives
//   dV = P^T dO,  dP = dO V^T,  D = rowsum(dO * O) (= rowsum(P * dP)),
//   dS = P * (dP - D),  dQ = scale dS K,  dK = scale dS^T Q,
// and a grouped key/value head sums over the query heads that read it.
//
// Three launches, no atomics:
//  * bwd_dvec_kernel: D for every (query, head), into the caller's workspace.
//  * attn_bwd_dq_kernel: per 128-query block, walks the key tiles like the
//    forward (S^T = K Q^T with Q in registers), also forms dP^T = V dO^T, and
//    accumulates dQ^T += K^T dS^T.
//  * attn_bwd_dkdv_kernel: per 128-key block (K and V in registers), walks the
//    query tiles of every query head of the group: S = Q K^T, dP = dO V^T,
//    dV^T += dO^T P, dK^T += Q^T dS.
// Tiles stream in by LDS DMA into the chunk-major layout of attn_device.h with
// rows permuted (key_of_row), so one tile serves both MFMA operand shapes: row
// fragments (16-byte reads, rows in key_of_row order: the scores come out in
// the order the P operand needs) and transposed fragments (ds_read_b64_tr_b16,
// rows in natural order through the same permutation).

#include "attn_internal.h"
#include "attn_device.h"

#include <math.h>
#include <stdlib.h>

namespace attnfwd {
namespace {

constexpr float kLog2e = 1.4426950408889634074f;

// Lane constants of the two fragment shapes of a 64 x D tile.
template <int D>
struct TileFrag {
  using L = PipeLayout<D>;
  int rd[2];  // row fragment: chunk parity 0 / 1
  int tr[2];  // transposed fragment: lower / upper 4 rows of an 8-row group
  __device__ __forceinline__ void init(int lane) {
    const int l32 = lane & 31, hh = lane >> 5;
    rd[0] = L::at(l32, hh, L::GK);
    rd[1] = L::at(l32, 2 + hh, L::GK);
    const int u = (lane & 15) >> 2;
    const int vcc = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    // natural row 8hh + u + 4hi sits at LDS row key_of_row(...) = 8hi + 4hh + u
    tr[0] = L::at(4 * hh + u, vcc, L::GK) + 8 * (lane & 1);
    tr[1] = L::at(8 + 4 * hh + u, vcc, L::GK) + 8 * (lane & 1);
  }
  // A operand rows 32 blk + 0..31 (LDS order), dims 16 s .. 16 s + 15
  __device__ __forceinline__ bf16x8 row(const unsigned char* t, int blk, int s) const {
    const int cst = (32 * blk / L::R) * L::GK + 16 * L::R * 2 * (s & ~1);
    return *reinterpret_cast<const bf16x8*>(t + rd[s & 1] + cst);
  }
  // A operand dims 32 db .. 32 db + 31 by rows 32 blk + 16 tt + 0..15 (natural)
  __device__ __forceinline__ bf16x8 trn(const unsigned char* t, int blk, int tt, int db) const {
    const int cst = ((32 * blk + 16 * tt) / L::R) * L::GK + 16 * L::R * 4 * db;
    const uint2 lo = ds_read_tr16(reinterpret_cast<const uint16_t*>(t + tr[0] + cst));
    const uint2 hi = ds_read_tr16(reinterpret_cast<const uint16_t*>(t + tr[1] + cst));
    return as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
  }
};

// DMA of rows r0 .. r0+ROWS-1 of a bf16 matrix (row pitch row_bytes, rows
// past the descriptor's range read as zero) into a ROWS-row tile (64 or 32)
// at LDS byte address tile, rows permuted within 32-row blocks; this wave
// issues instructions w, w + nw, ... of the tile's ROWS / R.
template <int D, int ROWS = 64>
__device__ __forceinline__ void dma_rows(u32x4 desc, uint32_t r0, uint32_t row_bytes, uint32_t tile,
                                         int w, int nw, int lane) {
  using L = PipeLayout<D>;
  constexpr int R = L::R;
  constexpr int NI = ROWS / R;
  const int c = lane / R;
  for (int q = w; q < NI; q += nw) {
    const int row = q * R + ((lane % R) ^ L::rot(c));
    const int src = (row & ~31) + key_of_row(row & 31);
    dma16(desc, (r0 + (uint32_t)src) * row_bytes + (uint32_t)c * 16,
          __builtin_amdgcn_readfirstlane(tile + q * L::GK));
  }
}

constexpr int kTileBytes128 = 16 * PipeLayout<128>::GK;

template <int D, int ROWS = 64>
constexpr int tile_bytes() { return (ROWS / PipeLayout<D>::R) * PipeLayout<D>::GK; }

// ---------------------------------------------------------------------------
// D = rowsum(dO * O) for every (query row, head): one wave per pair.
// ---------------------------------------------------------------------------
template <int D, bool VARLEN>
__global__ __launch_bounds__(256) void bwd_dvec_kernel(const AttnArgs a, const uint16_t* __restrict__ dout,
                                                       const int64_t n_pairs) {
  const int lane = threadIdx.x & 63;
  const int64_t pair = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (pair >= n_pairs) return;
  // pair -> (row, head); rows are packed tokens (varlen) or (batch, seq)
  const int h = (int)(pair % a.hq);
  const int64_t row = pair / a.hq;
  int64_t orow, lse_at;
  if constexpr (VARLEN) {
    orow = row;
    lse_at = (int64_t)h * a.lse_hs + row;
  } else {
    const int64_t b = row / a.sq, s = row - b * a.sq;
    orow = row;
    lse_at = b * a.lse_bs + (int64_t)h * a.lse_hs + s;
  }
  float acc = 0.f;
  for (int d = lane; d < D; d += 64) {
    const float o = a.o[orow * a.o_ss + (int64_t)h * a.o_hs + d];
    const uint16_t g = dout[orow * a.q_ss + (int64_t)h * a.q_hs + d];
    acc = fmaf(o, __uint_as_float((uint32_t)g << 16), acc);
  }
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (lane == 0) a.part_lse[lse_at] = acc;  // part_lse carries the D workspace here
}

// ---------------------------------------------------------------------------
// dQ: 4 waves x 32 queries; K/V tiles of 64 keys (32 at head_dim 256, where
// the score, dP and dS blocks of 64 keys would push Q, dO and dQ into spills)
// in two LDS buffers.
// ---------------------------------------------------------------------------
template <int D, bool VARLEN>
__global__ __launch_bounds__(256, D == 256 ? 1 : 2) void attn_bwd_dq_kernel(const AttnArgs a, const uint16_t* dout,
                                                            float* dq) {
  constexpr int BM = 128, BN = D == 256 ? 32 : 64;
  constexpr int NDS = D / 16, NDB = D / 32, NKB = BN / 32;
  constexpr int TB = tile_bytes<D, BN>();
  __shared__ __attribute__((aligned(16))) unsigned char lds[4 * TB];  // K0 V0 K1 V1
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  const int rows = a.nseq * a.hq;
  const int qb_rev = blockIdx.x / rows;
  const int p = blockIdx.x - qb_rev * rows;
  const int seq = p / a.hq, h = p - seq * a.hq;
  const int qb = a.causal ? (a.n_qb - 1 - qb_rev) : qb_rev;
  int lq, lk;
  int64_t qrow0, qoff, koff, voff, dvoff;
  if constexpr (VARLEN) {
    const SeqRows sr = seq_rows(a, seq);
    lq = sr.lq; lk = sr.lk;
    qrow0 = sr.q_row;
    koff = (int64_t)sr.k_row * a.k_ss;
    voff = (int64_t)sr.k_row * a.v_ss;
    dvoff = (int64_t)h * a.lse_hs + sr.qs;
  } else {
    lq = a.sq; lk = a.sk;
    qrow0 = (int64_t)seq * a.sq;
    koff = (int64_t)seq * a.k_bs;
    voff = (int64_t)seq * a.v_bs;
    dvoff = (int64_t)seq * a.lse_bs + (int64_t)h * a.lse_hs;
  }
  qoff = qrow0 * a.q_ss;
  const int q0 = qb * BM;
  if (q0 >= lq) return;
  const int kvh = h / a.group;
  const int off = lk - lq;
  int kend = lk;
  if (a.causal) kend = min(lk, q0 + BM + off);
  const int n_kt = kend > 0 ? (kend + BN - 1) / BN : 0;
  const int qw0 = q0 + wave * 32;
  int kend_w = lk;
  if (a.causal) kend_w = min(lk, qw0 + 32 + off);
  if (qw0 >= lq) kend_w = 0;

  // Q and dO of this wave's 32 queries as B operands (dims 16 s + 8 hh ..)
  const uint16_t* qbase = a.q + qoff + (int64_t)h * a.q_hs;
  const uint16_t* dobase = dout + qoff + (int64_t)h * a.q_hs;
  const __amdgpu_buffer_rsrc_t qrs = make_rsrc(qbase, span_bytes(lq, a.q_ss));
  const __amdgpu_buffer_rsrc_t drs = make_rsrc(dobase, span_bytes(lq, a.q_ss));
  bf16x8 qf[NDS], df[NDS];
  {
    const uint32_t ob = (uint32_t)(qw0 + l32) * (uint32_t)a.q_ss * 2 + hh * 16;
#pragma unroll
    for (int s = 0; s < NDS; ++s) {
      u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(qrs, (int)(ob + 32 * s), 0, 0);
      u32x4 y = __builtin_amdgcn_raw_buffer_load_b128(drs, (int)(ob + 32 * s), 0, 0);
      asm volatile("" : "+v"(x), "+v"(y));
      qf[s] = __builtin_bit_cast(bf16x8, x);
      df[s] = __builtin_bit_cast(bf16x8, y);
    }
  }
  // per-query constants: log2-domain LSE (+inf for a row with no key) and D
  const int qrow = qw0 + l32;
  float lse2 = INFINITY, dvec = 0.f;
  if (qrow < lq) {
    const float lv = a.lse[dvoff + qrow];
    lse2 = lv == -INFINITY ? INFINITY : lv * kLog2e;
    dvec = a.part_lse[dvoff + qrow];
  }

  const uint32_t k_rb = (uint32_t)a.k_ss * 2, v_rb = (uint32_t)a.v_ss * 2;
  const u32x4 kdesc = make_desc(a.k + koff + (int64_t)kvh * a.k_hs, span_bytes(lk, a.k_ss));
  const u32x4 vdesc = make_desc(a.v + voff + (int64_t)kvh * a.v_hs, span_bytes(lk, a.v_ss));
  const uint32_t lds0 = lds_addr(lds);
  auto dma = [&](int t) {
    const uint32_t b = (uint32_t)(t & 1) * 2 * TB;
    dma_rows<D, BN>(kdesc, (uint32_t)t * BN, k_rb, lds0 + b, wave, 4, lane);
    dma_rows<D, BN>(vdesc, (uint32_t)t * BN, v_rb, lds0 + b + TB, wave, 4, lane);
  };
  TileFrag<D> fr;
  fr.init(lane);

  f32x16 dqacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dqacc[db] = f32x16{};

  if (n_kt > 0) dma(0);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __syncthreads();
  for (int t = 0; t < n_kt; ++t) {
    if (t + 1 < n_kt) dma(t + 1);
    const int kbeg = t * BN;
    if (kbeg < kend_w) {
      const unsigned char* kt = lds + (t & 1) * 2 * TB;
      const unsigned char* vt = kt + TB;
      f32x16 st[NKB], pt[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int s = 0; s < NDS; ++s) {
          st[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr.row(kt, kb, s), qf[s],
                                                           s == 0 ? f32x16{} : st[kb], 0, 0, 0);
          pt[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr.row(vt, kb, s), df[s],
                                                           s == 0 ? f32x16{} : pt[kb], 0, 0, 0);
        }
      const bool edge = (kbeg + BN > lk) || (a.causal && kbeg + BN - 1 > qw0 + off);
      const int lim = a.causal ? min(lk - 1, qrow + off) : lk - 1;
      bf16x8 dsf[NKB][2];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float s = st[kb][r] * a.c - lse2;
          if (edge) {
            const int key = kbeg + kb * 32 + ((r >> 3) << 4) + hh * 8 + (r & 7);
            if (key > lim) s = -INFINITY;
          }
          const float pv = __builtin_amdgcn_exp2f(s);
          st[kb][r] = pv * (pt[kb][r] - dvec);
        }
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          uint4 w;
          w.x = pack_bf16x2(st[kb][8 * tt + 0], st[kb][8 * tt + 1]);
          w.y = pack_bf16x2(st[kb][8 * tt + 2], st[kb][8 * tt + 3]);
          w.z = pack_bf16x2(st[kb][8 * tt + 4], st[kb][8 * tt + 5]);
          w.w = pack_bf16x2(st[kb][8 * tt + 6], st[kb][8 * tt + 7]);
          dsf[kb][tt] = as_bf16x8(w);
        }
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int tt = 0; tt < 2; ++tt)
            dqacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr.trn(kt, kb, tt, db), dsf[kb][tt],
                                                                dqacc[db], 0, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();
  }

  if (qrow < lq) {
    const float sc = a.c / kLog2e;  // the softmax scale
    float* op = dq + ((qrow0 + qrow) * a.hq + h) * D + hh * 4;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float4 w;
        w.x = dqacc[db][4 * g + 0] * sc;
        w.y = dqacc[db][4 * g + 1] * sc;
        w.z = dqacc[db][4 * g + 2] * sc;
        w.w = dqacc[db][4 * g + 3] * sc;
        *reinterpret_cast<float4*>(op + db * 32 + 8 * g) = w;
      }
  }
}

// ---------------------------------------------------------------------------
// dK, dV: 4 waves x 32 keys; Q/dO tiles of 64 queries in two LDS buffers,
// walked for every query head of the group.
// ---------------------------------------------------------------------------
// MODE 0: dK and dV together; 1: dV only (S and P^T dO); 2: dK only (S, dP
// and Q^T dS).  The split modes hold fewer registers per wave, so more waves
// share a SIMD, at the price of computing S in both.
template <int D, bool VARLEN, int MODE>
__global__ __launch_bounds__(256, D == 256 ? 1 : (MODE == 1 ? 3 : (MODE == 2 ? 2 : (D >= 128 ? 1 : 2))))
void attn_bwd_dkdv_kernel(const AttnArgs a, const uint16_t* dout, float* dk, float* dv, int n_kb) {
  constexpr bool DO_DK = MODE != 1, DO_DV = MODE != 2;
  constexpr int BKEYS = 128, BQ = 64;
  constexpr int NDS = D / 16, NDB = D / 32;
  constexpr int TB = tile_bytes<D>();
  __shared__ __attribute__((aligned(16))) unsigned char lds[4 * TB];  // Q0 dO0 Q1 dO1
  __shared__ __attribute__((aligned(16))) float vec[2][2][BQ];       // [buf][lse2 | D][query]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  const int krows = a.nseq * a.hkv;
  const int kb_rev = blockIdx.x / krows;
  const int p = blockIdx.x - kb_rev * krows;
  const int seq = p / a.hkv, kvh = p - seq * a.hkv;
  const int kblk = a.causal ? kb_rev : (n_kb - 1 - kb_rev);  // causal: early keys see the most queries
  int lq, lk;
  int64_t qoff, koff, voff, kout, lsebase;
  if constexpr (VARLEN) {
    const SeqRows sr = seq_rows(a, seq);
    lq = sr.lq; lk = sr.lk;
    qoff = (int64_t)sr.q_row * a.q_ss;
    koff = (int64_t)sr.k_row * a.k_ss;
    voff = (int64_t)sr.k_row * a.v_ss;
    kout = (int64_t)sr.k_row;
    lsebase = sr.qs;
  } else {
    lq = a.sq; lk = a.sk;
    qoff = (int64_t)seq * a.q_bs;
    koff = (int64_t)seq * a.k_bs;
    voff = (int64_t)seq * a.v_bs;
    kout = (int64_t)seq * a.sk;
    lsebase = (int64_t)seq * a.lse_bs;
  }
  const int k0 = kblk * BKEYS;
  if (k0 >= lk) return;
  const int off = lk - lq;
  const int kw0 = k0 + wave * 32;
  const int key = kw0 + l32;  // this lane's key column

  // K and V of this wave's 32 keys as B operands (dims 16 s + 8 hh ..)
  const uint16_t* kbase = a.k + koff + (int64_t)kvh * a.k_hs;
  const uint16_t* vbase = a.v + voff + (int64_t)kvh * a.v_hs;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(kbase, span_bytes(lk, a.k_ss));
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vbase, span_bytes(lk, a.v_ss));
  // Fused pass at head_dim 128: K and V (64 registers) go to the accumulation
  // registers, which MFMAs read as operands directly, so the vector registers
  // hold the dK/dV accumulators and the S/dP blocks without spilling.
  constexpr bool KV_IN_ACC = D == 128 && MODE == 0;
  auto to_acc = [](u32x4 x) __attribute__((always_inline)) {
    u32x4 r;
#pragma unroll
    for (int k = 0; k < 4; ++k) asm volatile("v_accvgpr_write_b32 %0, %1" : "=a"(r[k]) : "v"(x[k]));
    return r;
  };
  bf16x8 kf[NDS], vf[NDS];
  {
    const uint32_t kb_ = (uint32_t)key * (uint32_t)a.k_ss * 2 + hh * 16;
    const uint32_t vb_ = (uint32_t)key * (uint32_t)a.v_ss * 2 + hh * 16;
#pragma unroll
    for (int s = 0; s < NDS; ++s) {
      u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(krs, (int)(kb_ + 32 * s), 0, 0);
      asm volatile("" : "+v"(x));
      if constexpr (KV_IN_ACC) x = to_acc(x);
      kf[s] = __builtin_bit_cast(bf16x8, x);
      if constexpr (DO_DK) {
        u32x4 y = __builtin_amdgcn_raw_buffer_load_b128(vrs, (int)(vb_ + 32 * s), 0, 0);
        asm volatile("" : "+v"(y));
        if constexpr (KV_IN_ACC) y = to_acc(y);
        vf[s] = __builtin_bit_cast(bf16x8, y);
      }
    }
    if constexpr (KV_IN_ACC) asm volatile("s_nop 7");
  }

  // query tiles: those with a query that sees a key of this block, per head
  const int first_q = a.causal ? max(0, k0 - off) : 0;
  const int qt0 = first_q / BQ;
  const int n_qt_all = lq > 0 ? (lq + BQ - 1) / BQ : 0;
  const int nq = max(n_qt_all - qt0, 0);
  const int n_tiles = nq * a.group;

  const uint32_t q_rb = (uint32_t)a.q_ss * 2;
  const uint32_t lds0 = lds_addr(lds);
  TileFrag<D> fr;
  fr.init(lane);

  auto tile_head = [&](int t) { return kvh * a.group + t / nq; };
  auto tile_q0 = [&](int t) { return (qt0 + t % nq) * BQ; };
  auto dma = [&](int t) {
    const int hq = tile_head(t);
    const uint32_t b = (uint32_t)(t & 1) * 2 * TB;
    const u32x4 qd = make_desc(a.q + qoff + (int64_t)hq * a.q_hs, span_bytes(lq, a.q_ss));
    const u32x4 dd = make_desc(dout + qoff + (int64_t)hq * a.q_hs, span_bytes(lq, a.q_ss));
    dma_rows<D>(qd, (uint32_t)tile_q0(t), q_rb, lds0 + b, wave, 4, lane);
    dma_rows<D>(dd, (uint32_t)tile_q0(t), q_rb, lds0 + b + TB, wave, 4, lane);
  };
  // lse2 and D of the tile's 64 queries (threads 0..63 and 64..127)
  auto vec_load = [&](int t, float& x) {
    const int hq = tile_head(t);
    const int i = tile_q0(t) + (tid & 63);
    x = 0.f;
    if (tid < 128 && i < lq) {
      const int64_t at = lsebase + (int64_t)hq * a.lse_hs + i;
      if (tid < 64) {
        const float lv = a.lse[at];
        x = lv == -INFINITY ? INFINITY : lv * kLog2e;
      } else {
        x = a.part_lse[at];
      }
    } else if (tid < 64) {
      x = INFINITY;  // rows past the sequence: P = 0
    }
  };

  f32x16 dkacc[NDB], dvacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    dkacc[db] = f32x16{};
    dvacc[db] = f32x16{};
  }

  float xv;
  if (n_tiles > 0) {
    dma(0);
    vec_load(0, xv);
    if (tid < 128) vec[0][tid >> 6][tid & 63] = xv;
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __syncthreads();
  for (int t = 0; t < n_tiles; ++t) {
    if (t + 1 < n_tiles) {
      dma(t + 1);
      vec_load(t + 1, xv);
    }
    const int iq0 = tile_q0(t);
    const unsigned char* qt = lds + (t & 1) * 2 * TB;
    const unsigned char* dt = qt + TB;
    const float* lsev = vec[t & 1][0];
    const float* dvv = vec[t & 1][1];
#pragma unroll
    for (int blk = 0; blk < BQ / 32; ++blk) {
      f32x16 s_acc = f32x16{}, p_acc = f32x16{};
#pragma unroll
      for (int s = 0; s < NDS; ++s) {
        s_acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr.row(qt, blk, s), kf[s], s_acc, 0, 0, 0);
        if constexpr (DO_DK)
          p_acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr.row(dt, blk, s), vf[s], p_acc, 0, 0, 0);
      }
      // register r = 8 tt + e holds query iq0 + 32 blk + 16 tt + 8 hh + e.
      // Only the causal test needs evaluating, and only on tiles that cross
      // the diagonal: queries past the sequence (and rows with no visible key)
      // carry LSE = +inf, so their P is 0; a key past the sequence only feeds
      // its own dK/dV column, which is never stored.
      const bool diag = a.causal && (kw0 + 31 > iq0 + 32 * blk + off);
      bf16x8 pf[2], dsf[2];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int qi = 32 * blk + 16 * tt + 8 * hh;
        const float4 l0 = *reinterpret_cast<const float4*>(lsev + qi);
        const float4 l1 = *reinterpret_cast<const float4*>(lsev + qi + 4);
        const float4 d0 = *reinterpret_cast<const float4*>(dvv + qi);
        const float4 d1 = *reinterpret_cast<const float4*>(dvv + qi + 4);
        const float lz[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
        const float dz[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
        float pv[8], dsv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int r = 8 * tt + e;
          const int i = iq0 + qi + e;
          float x = fmaf(s_acc[r], a.c, -lz[e]);
          if (diag && key > i + off) x = -INFINITY;
          pv[e] = __builtin_amdgcn_exp2f(x);
          if constexpr (DO_DK) dsv[e] = pv[e] * (p_acc[r] - dz[e]);
        }
        uint4 w;
        if constexpr (DO_DV) {
          w.x = pack_bf16x2(pv[0], pv[1]);
          w.y = pack_bf16x2(pv[2], pv[3]);
          w.z = pack_bf16x2(pv[4], pv[5]);
          w.w = pack_bf16x2(pv[6], pv[7]);
          pf[tt] = as_bf16x8(w);
        }
        if constexpr (DO_DK) {
          w.x = pack_bf16x2(dsv[0], dsv[1]);
          w.y = pack_bf16x2(dsv[2], dsv[3]);
          w.z = pack_bf16x2(dsv[4], dsv[5]);
          w.w = pack_bf16x2(dsv[6], dsv[7]);
          dsf[tt] = as_bf16x8(w);
        }
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          if constexpr (DO_DV)
            dvacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr.trn(dt, blk, tt, db), pf[tt],
                                                                dvacc[db], 0, 0, 0);
          if constexpr (DO_DK)
            dkacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr.trn(qt, blk, tt, db), dsf[tt],
                                                                dkacc[db], 0, 0, 0);
        }
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    if (t + 1 < n_tiles && tid < 128) vec[(t + 1) & 1][tid >> 6][tid & 63] = xv;
    __syncthreads();
  }

  if (key < lk) {
    const float sc = a.c / kLog2e;
    const int64_t rowi = (kout + key) * (int64_t)a.hkv + kvh;  // (row, head) of dk / dv
    float* kp = dk + rowi * D + hh * 4;
    float* vp = dv + rowi * D + hh * 4;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float4 w, u;
        w.x = dkacc[db][4 * g + 0] * sc;
        w.y = dkacc[db][4 * g + 1] * sc;
        w.z = dkacc[db][4 * g + 2] * sc;
        w.w = dkacc[db][4 * g + 3] * sc;
        u.x = dvacc[db][4 * g + 0];
        u.y = dvacc[db][4 * g + 1];
        u.z = dvacc[db][4 * g + 2];
        u.w = dvacc[db][4 * g + 3];
        if constexpr (DO_DK) *reinterpret_cast<float4*>(kp + db * 32 + 8 * g) = w;
        if constexpr (DO_DV) *reinterpret_cast<float4*>(vp + db * 32 + 8 * g) = u;
      }
  }
}

// ATTN_BWD_SPLIT=1 runs dV and dK as two passes (sweeps); the default is the
// fused pass, measured faster at every head dim it serves (cold, same process:
// 1x8192 causal d=128 1203 us fused vs 1337 split; 4096 causal d=64 639 vs
// 792 us, d=32 817 vs 1037 us).
int bwd_split_mode(int) {
  const char* s = getenv("ATTN_BWD_SPLIT");
  return (s != nullptr && s[0] == '1' && s[1] == '\0') ? 1 : 0;
}

template <int D, bool VARLEN>
hipError_t bwd_d(const AttnArgs& a, const uint16_t* dout, float* dq, float* dk, float* dv,
                 int64_t n_pairs, int n_kb, hipStream_t stream) {
  const int64_t gd = (n_pairs + 3) / 4;
  const int64_t gq = (int64_t)a.nseq * a.hq * a.n_qb;
  const int64_t gk = (int64_t)a.nseq * a.hkv * n_kb;
  if (gd > 0x7fffffff || gq > 0x7fffffff || gk > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (gd > 0)
    hipLaunchKernelGGL((bwd_dvec_kernel<D, VARLEN>), dim3((unsigned)gd), dim3(256), 0, stream, a, dout,
                       n_pairs);
  if (gq > 0)
    hipLaunchKernelGGL((attn_bwd_dq_kernel<D, VARLEN>), dim3((unsigned)gq), dim3(256), 0, stream, a,
                       dout, dq);
  if (gk > 0) {
    // head_dim 256: the fused pass would need K, V, dK and dV of 32 keys (512
    // registers) and spills; the two passes fit one wave per SIMD.
    if (D == 256 || bwd_split_mode(D)) {
      hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, VARLEN, 1>), dim3((unsigned)gk), dim3(256), 0,
                         stream, a, dout, dk, dv, n_kb);
      hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, VARLEN, 2>), dim3((unsigned)gk), dim3(256), 0,
                         stream, a, dout, dk, dv, n_kb);
    } else if constexpr (D != 256) {
      hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, VARLEN, 0>), dim3((unsigned)gk), dim3(256), 0,
                         stream, a, dout, dk, dv, n_kb);
    }
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention_bwd(const AttnArgs& a, int head_dim, bool varlen, const uint16_t* dout,
                                float* dq, float* dk, float* dv, int64_t n_pairs, int n_kb,
                                hipStream_t stream) {
  switch (head_dim) {
    case 32: return varlen ? bwd_d<32, true>(a, dout, dq, dk, dv, n_pairs, n_kb, stream)
                           : bwd_d<32, false>(a, dout, dq, dk, dv, n_pairs, n_kb, stream);
    case 64: return varlen ? bwd_d<64, true>(a, dout, dq, dk, dv, n_pairs, n_kb, stream)
                           : bwd_d<64, false>(a, dout, dq, dk, dv, n_pairs, n_kb, stream);
    case 128: return varlen ? bwd_d<128, true>(a, dout, dq, dk, dv, n_pairs, n_kb, stream)
                            : bwd_d<128, false>(a, dout, dq, dk, dv, n_pairs, n_kb, stream);
    case 256: return varlen ? bwd_d<256, true>(a, dout, dq, dk, dv, n_pairs, n_kb, stream)
                            : bwd_d<256, false>(a, dout, dq, dk, dv, n_pairs, n_kb, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace attnfwd
