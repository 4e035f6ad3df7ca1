// FlashAttention forward for gfx950 (MI355X), hand-written HIP.
//
// What is computed (page "Intro to FlashAttention on Ascend CANN"): for every
// (sequence, query head) O = softmax(scale * Q K^T) V, tiled so the score matrix
// never leaves the chip ("tiled computation"), with the online softmax that
// carries a running row maximum m and row sum l across key blocks and rescales
// the partial output when m grows ("the first pitfall"), and with causal
// blocks skipped instead of masked after the fact (paragraph on the fused
// causal mask).  The row sum/maximum bookkeeping runs in base 2: scores are
// multiplied by c = scale * log2(e) so that exp becomes the hardware exp2.
//
// Mapping onto CDNA4:
//  * A workgroup owns BM = waves * 32 * qcols consecutive queries of one
//    (sequence, head); each wave owns 32 * qcols of them.
//  * Scores are produced transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: K (32 keys x 16 dims) is the A operand read
//    from LDS, Q^T is the B operand held in registers for the whole loop.  In
//    the 32x32 accumulator layout each lane then holds one query's column, 16
//    keys of it, and the other 16 keys sit in lane ^ 32.  Row max and row sum
//    are therefore in-lane reductions plus one v_permlane32_swap.
//  * The K rows fed to the A operand are permuted (key_of_row) so that lane
//    half h, accumulator registers 8t..8t+7 hold keys 16t + 8h + 0..7.  Those
//    8 probabilities, rounded to bf16, are exactly the B operand of the second
//    product O^T += V^T P^T for keys 16t..16t+15: P never leaves registers.
//  * Three kernel families share that mapping.  The staged kernel
//    (attn_fwd_kernel) moves K/V tiles HBM -> registers -> LDS and stores V
//    transposed (V^T[d][key]), so the A operand of the second product (32 dims
//    x 8 consecutive keys per lane) is one 16-byte LDS read; the global loads
//    of the next tile are issued before the current tile's math.  The
//    DMA-staged kernel (attn_fwd_dma_kernel) moves tiles HBM -> LDS directly
//    and reads V row-major through the transposing LDS read.  The
//    software-pipelined kernel (attn_fwd_pipe_kernel) adds an LDS layout with
//    additive fragment addresses and overlaps the scores of the next tile
//    with the softmax of the current one inside each wave.
//  * Causal: key tiles beyond the diagonal of the whole query block are never
//    loaded; a wave whose queries all precede a tile skips its math; only
//    tiles that cross the diagonal (or the sequence end) apply a mask.
//  * Grid: one workgroup per (query block, sequence, head).  For causal work
//    the query-block index runs from the last (most key tiles) to the first, so
//    the longest workgroups are dispatched first.  Rows of (sequence, head)
//    are remapped so that each XCD (workgroups are dealt round-robin over 8)
//    receives a contiguous range of heads, which keeps the K/V of grouped heads
//    in one L2.

#include "attn_internal.h"
#include "attn_device.h"

#include <math.h>

#include <type_traits>

namespace attnfwd {
namespace {

// Online-softmax rescale threshold in base-2 units.  The running row
// maximum m used as the exp2 reference is only raised when a new tile's
// maximum exceeds it by more than this; until then p = 2^(c*s - m) stays below
// 2^8, far inside fp32 and bf16 range.  The final O / l and LSE = m + log2 l
// are exact for whatever m was used, so skipping small rescales changes no
// result beyond rounding, and it removes the per-tile pass over O.
constexpr float kRescaleThreshold = 8.0f;

// LDS fragment reads kept in flight ahead of the MFMA that consumes them.
constexpr int kLdsAhead = 6;

// Scheduling hint for a straight-line run of N (LDS read, MFMA) pairs: issue
// kLdsAhead reads first, then alternate MFMA / read, so each MFMA finds its
// operand already loaded instead of waiting out the LDS latency.
template <int N>
__device__ __forceinline__ void lds_pipeline_hint() {
  constexpr int A = N < kLdsAhead ? N : kLdsAhead;
  __builtin_amdgcn_sched_group_barrier(0x100, A, 0);
#pragma unroll
  for (int i = 0; i < N - A; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, A, 0);
}

// Kernel variant flags.
constexpr int kPrio = 1;  // raise wave priority while issuing MFMA blocks

// KG > 1 splits the key range of a query block over KG groups of waves: the
// waves of group g take tiles g, g+KG, g+2KG, ... of the block, so a block's
// serial key loop is KG times shorter (this is what keeps few-head, long
// causal sequences from being bound by their last query block).  Each group
// keeps its own (m, l, O); at the end the groups merge through LDS with the
// same rescaling rule as the online softmax.
template <int D, int BN, int WAVES, int QC, int MINW, bool VARLEN, int FLAGS = 0, int KG = 1>
__global__ __launch_bounds__(WAVES * 64, MINW) void attn_fwd_kernel(const AttnArgs a) {
  constexpr int NT = WAVES * 64;
  constexpr int QW = WAVES / KG;  // waves per key group (they split the queries)
  static_assert(WAVES % KG == 0, "key groups must split the waves evenly");
  constexpr int SUB = (D == 256 || BN == 32) ? 32 : 64;  // keys per softmax sub-block
  constexpr int NSB = BN / SUB;
  static_assert(BN % SUB == 0, "tile must hold whole sub-blocks");
  constexpr int BM = QW * 32 * QC;
  constexpr int PAD = 8;            // bf16 elements of padding per LDS row
  constexpr int KS = D + PAD;       // K tile row stride (keys are rows)
  constexpr int VS = BN + PAD;      // V^T tile row stride (dims are rows)
  constexpr int KT_ELEMS = BN * KS;
  constexpr int VT_ELEMS = D * VS;
  constexpr int NKB = SUB / 32;     // 32-key blocks per sub-block
  constexpr int NDS = D / 16;       // 16-dim slices of one key row
  constexpr int NDB = D / 32;       // 32-dim blocks of the output
  constexpr int K_TILE_UNITS = BN * D / 8;          // 16-byte chunks of a K tile
  constexpr int K_UNITS = KG * K_TILE_UNITS;         // ... of the KG tiles of one step
  constexpr int K_PER = (K_UNITS + NT - 1) / NT;
  constexpr int V_TILE_UNITS = (BN / 4) * (D / 8);  // 4 keys x 8 dims units of a V tile
  constexpr int V_UNITS = KG * V_TILE_UNITS;
  constexpr int V_PER = (V_UNITS + NT - 1) / NT;
  static_assert(BN % 32 == 0 && D % 32 == 0, "tile shape");

  // Two buffers of KG K/V^T tiles: step i+1 is written while step i is read.
  // One allocation, so the key-group merge can reuse all of it.
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * KG * (KT_ELEMS + VT_ELEMS)];
  uint16_t* const ks = smem;
  uint16_t* const vt = smem + 2 * KG * KT_ELEMS;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kg = wave / QW;     // key group of this wave
  const int qw = wave - kg * QW;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  // ---- tile decode ------------------------------------------------------
  const int rows = a.nseq * a.hq;
  const int id = blockIdx.x;
  const int qb_rev = id / rows;
  int p = id - qb_rev * rows;
  if (a.xcd_remap) p = (p & 7) * (rows >> 3) + (p >> 3);
  const int seq = p / a.hq;
  const int h = p - seq * a.hq;
  const int qb = a.causal ? (a.n_qb - 1 - qb_rev) : qb_rev;

  int lq, lk;
  int64_t qoff, koff, voff, ooff, lseoff;
  if constexpr (VARLEN) {
    const SeqRows sr = seq_rows(a, seq);
    lq = sr.lq;
    lk = sr.lk;
    qoff = (int64_t)sr.q_row * a.q_ss;
    koff = (int64_t)sr.k_row * a.k_ss;
    voff = (int64_t)sr.k_row * a.v_ss;
    ooff = (int64_t)sr.q_row * a.o_ss;
    lseoff = sr.qs;
  } else {
    lq = a.sq;
    lk = a.sk;
    qoff = (int64_t)seq * a.q_bs;
    koff = (int64_t)seq * a.k_bs;
    voff = (int64_t)seq * a.v_bs;
    ooff = (int64_t)seq * a.o_bs;
    lseoff = (int64_t)seq * a.lse_bs;
  }
  const int q0 = qb * BM;
  if (q0 >= lq) return;
  const int kvh = h / a.group;
  const uint16_t* qbase = a.q + qoff + (int64_t)h * a.q_hs;
  const uint16_t* kbase = a.k + koff + (int64_t)kvh * a.k_hs;
  const uint16_t* vbase = a.v + voff + (int64_t)kvh * a.v_hs;
  float* obase = a.o + ooff + (int64_t)h * a.o_hs;

  const int off = lk - lq;  // causal alignment: key j visible to query i iff j <= i + off
  int kend = lk;
  if (a.causal) kend = min(lk, q0 + BM + off);
  const int n_kt = kend > 0 ? (kend + BN - 1) / BN : 0;
  const int n_steps = (n_kt + KG - 1) / KG;

  const int qw0 = q0 + qw * 32 * QC;  // first query of this wave
  int kend_w = lk;
  if (a.causal) kend_w = min(lk, qw0 + 32 * QC + off);
  if (qw0 >= lq) kend_w = 0;  // a wave made only of padding rows does no math

  // ---- Q^T fragments (B operand), kept in registers ----------------------
  const __amdgpu_buffer_rsrc_t qrs = make_rsrc(qbase, span_bytes(lq, a.q_ss));
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(kbase, span_bytes(lk, a.k_ss));
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vbase, span_bytes(lk, a.v_ss));
  const uint32_t k_row_bytes = (uint32_t)a.k_ss * 2;
  const uint32_t v_row_bytes = (uint32_t)a.v_ss * 2;
  u32x4 qraw[QC][NDS];
#pragma unroll
  for (int c = 0; c < QC; ++c) {
    const int qrow = qw0 + c * 32 + l32;  // rows past lq read as zeros
    const uint32_t qoff_b = (uint32_t)qrow * (uint32_t)a.q_ss * 2 + hh * 16;
#pragma unroll
    for (int s = 0; s < NDS; ++s)
      qraw[c][s] = __builtin_amdgcn_raw_buffer_load_b128(qrs, (int)(qoff_b + 32 * s), 0, 0);
  }
  // Empty asm that "redefines" the loaded registers: the compiler waits for the
  // Q loads once, here, instead of treating Q as in flight inside the key loop
  // (where its wait would also drain the K/V prefetch on every iteration).
  bf16x8 qf[QC][NDS];
#pragma unroll
  for (int c = 0; c < QC; ++c)
#pragma unroll
    for (int s = 0; s < NDS; ++s) {
      asm volatile("" : "+v"(qraw[c][s]));
      qf[c][s] = __builtin_bit_cast(bf16x8, q_sign(qraw[c][s], a.q_xor, a.q_clear));
    }

  f32x16 oacc[QC][NDB];
  float m_run[QC], l_run[QC];
#pragma unroll
  for (int c = 0; c < QC; ++c) {
    m_run[c] = -INFINITY;
    l_run[c] = 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[c][db] = f32x16{};
  }

  // ---- staging registers for the next K/V tile ----------------------------
  uint4 kreg[K_PER];
  uint4 vreg[V_PER][4];

  // Unit u of a step covers tile (step * KG + u / TILE_UNITS); its K rows
  // are consecutive keys, so a step's KG tiles are KG * BN consecutive keys.
  auto fetch = [&](int step) {
    const uint32_t kbeg = step * KG * BN;
#pragma unroll
    for (int i = 0; i < K_PER; ++i) {
      const int u = tid + i * NT;
      if (K_UNITS % NT == 0 || u < K_UNITS) {
        const uint32_t row = u / (D / 8);  // row within the step's KG * BN keys
        const uint32_t col = (u % (D / 8)) * 8;
        kreg[i] = buf_ld16(krs, (kbeg + row) * k_row_bytes + col * 2);
      }
    }
#pragma unroll
    for (int i = 0; i < V_PER; ++i) {
      const int u = tid + i * NT;
      if (V_UNITS % NT == 0 || u < V_UNITS) {
        const uint32_t g = u / V_TILE_UNITS;
        const uint32_t w = u - g * V_TILE_UNITS;
        const uint32_t kq = w % (BN / 4);
        const uint32_t dq = w / (BN / 4);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          vreg[i][j] = buf_ld16(vrs, (kbeg + g * BN + kq * 4 + j) * v_row_bytes + dq * 16);
      }
    }
  };

  auto stage = [&](int buf) {
    uint16_t* kd = ks + buf * KG * KT_ELEMS;  // KG tiles back to back: rows continue
#pragma unroll
    for (int i = 0; i < K_PER; ++i) {
      const int u = tid + i * NT;
      if (K_UNITS % NT == 0 || u < K_UNITS) {
        const int row = u / (D / 8);
        const int col = (u % (D / 8)) * 8;
        *reinterpret_cast<uint4*>(kd + row * KS + col) = kreg[i];
      }
    }
#pragma unroll
    for (int i = 0; i < V_PER; ++i) {
      const int u = tid + i * NT;
      if (V_UNITS % NT == 0 || u < V_UNITS) {
        const int g = u / V_TILE_UNITS;
        const int w = u - g * V_TILE_UNITS;
        uint16_t* vd = vt + (buf * KG + g) * VT_ELEMS;
        const int kq = w % (BN / 4);
        const int dq = w / (BN / 4);
        const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&vreg[i][0]);
        const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&vreg[i][1]);
        const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&vreg[i][2]);
        const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&vreg[i][3]);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          // dims dq*8+e of keys kq*4 .. kq*4+3 -> 4 consecutive bf16 of a V^T row
          const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
          uint2 out;
          out.x = __builtin_amdgcn_perm(w1[e >> 1], w0[e >> 1], sel);
          out.y = __builtin_amdgcn_perm(w3[e >> 1], w2[e >> 1], sel);
          *reinterpret_cast<uint2*>(vd + (dq * 8 + e) * VS + kq * 4) = out;
        }
      }
    }
  };

  if (n_steps > 0) {
    fetch(0);
    stage(0);
  }
  __syncthreads();

  for (int step = 0; step < n_steps; ++step) {
    const int buf = step & 1;
    if (step + 1 < n_steps) fetch(step + 1);
    const int kt = step * KG + kg;  // the tile this wave's group handles

#pragma unroll
    for (int sb = 0; sb < NSB; ++sb) {
    const int kbeg = kt * BN + sb * SUB;
    if (kbeg < kend_w) {
      const uint16_t* kd = ks + (buf * KG + kg) * KT_ELEMS + sb * SUB * KS;
      const uint16_t* vd = vt + (buf * KG + kg) * VT_ELEMS + sb * SUB;
      // ---- S^T = K Q^T ------------------------------------------------------
      if constexpr (FLAGS & kPrio) __builtin_amdgcn_s_setprio(1);
      f32x16 sacc[QC][NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const uint16_t* kr = kd + (kb * 32 + key_of_row(l32)) * KS + hh * 8;
#pragma unroll
        for (int s = 0; s < NDS; ++s) {
          const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kr + 16 * s);
#pragma unroll
          for (int c = 0; c < QC; ++c)
            sacc[c][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                kf, qf[c][s], s == 0 ? f32x16{} : sacc[c][kb], 0, 0, 0);
        }
      }
      if constexpr (QC == 1) lds_pipeline_hint<NKB * NDS>();
      if constexpr (FLAGS & kPrio) __builtin_amdgcn_s_setprio(0);

      // ---- mask (only sub-blocks crossing the diagonal or the sequence end) --
      const bool need_mask = (kbeg + SUB > lk) || (a.causal && kbeg + SUB - 1 > qw0 + off);
      if (need_mask) {
        keep_branch();
#pragma unroll
        for (int c = 0; c < QC; ++c) {
          const int qi = qw0 + c * 32 + l32;
          const int lim = a.causal ? min(lk - 1, qi + off) : lk - 1;  // last visible key
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb) mask_block(sacc[c][kb], lim - kbeg - kb * 32 - hh * 8);
        }
      }

      // ---- online softmax (base 2, lazy rescale) ----------------------------
      bf16x8 pf[QC][NKB][2];
#pragma unroll
      for (int c = 0; c < QC; ++c) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[c][kb][r]);
        mx = half_max(mx);
        const float cand = mx * a.c;
        const bool grow = cand > m_run[c] + kRescaleThreshold;
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {
          // Only lanes whose own maximum grew move their reference; the others
          // scale by exactly 1, so a row's result never depends on its
          // neighbours in the wave.  A lane can only grow from a finite cand,
          // and m_run = -inf then gives alpha = 0.
          const float m_new = grow ? cand : m_run[c];
          const float alpha = grow ? __builtin_amdgcn_exp2f(m_run[c] - m_new) : 1.0f;
          m_run[c] = m_new;
          l_run[c] *= alpha;
#pragma unroll
          for (int db = 0; db < NDB; ++db) oacc[c][db] *= alpha;
        }
        const float m_use = (m_run[c] == -INFINITY) ? 0.f : m_run[c];
        float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float pv = __builtin_amdgcn_exp2f(fmaf(sacc[c][kb][r], a.c, -m_use));
            sacc[c][kb][r] = pv;
            if (r & 1) rs1 += pv; else rs0 += pv;
          }
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            uint4 u;
            u.x = pack_bf16x2(sacc[c][kb][8 * t + 0], sacc[c][kb][8 * t + 1]);
            u.y = pack_bf16x2(sacc[c][kb][8 * t + 2], sacc[c][kb][8 * t + 3]);
            u.z = pack_bf16x2(sacc[c][kb][8 * t + 4], sacc[c][kb][8 * t + 5]);
            u.w = pack_bf16x2(sacc[c][kb][8 * t + 6], sacc[c][kb][8 * t + 7]);
            pf[c][kb][t] = as_bf16x8(u);
          }
        }
        l_run[c] += rs0 + rs1;
      }

      // ---- O^T += V^T P^T ---------------------------------------------------
      if constexpr (FLAGS & kPrio) __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const uint16_t* vr = vd + (db * 32 + l32) * VS + hh * 8;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const bf16x8 vf = *reinterpret_cast<const bf16x8*>(vr + kb * 32 + 16 * t);
#pragma unroll
            for (int c = 0; c < QC; ++c)
              oacc[c][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[c][kb][t], oacc[c][db], 0, 0, 0);
          }
        }
      }
      if constexpr (QC == 1) lds_pipeline_hint<NDB * NKB * 2>();
      if constexpr (FLAGS & kPrio) __builtin_amdgcn_s_setprio(0);
    }
    }
    if (step + 1 < n_steps) stage(buf ^ 1);
    __syncthreads();
  }

  // ---- merge of the key groups (KG > 1) through LDS -------------------------
  if constexpr (KG > 1) {
    constexpr int NREG = QC * (NDB * 16 + 2);  // O accumulators, m, l per lane
    static_assert((KG - 1) * QW * NREG * 64 * 4 <= 2 * KG * (KT_ELEMS + VT_ELEMS) * 2,
                  "merge buffer must fit in the tile buffers");
    float* mrg = reinterpret_cast<float*>(smem);  // [slot][reg][lane]; the key loop is over
    if (kg > 0) {
      float* dst = mrg + ((kg - 1) * QW + qw) * NREG * 64 + lane;
#pragma unroll
      for (int c = 0; c < QC; ++c) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) dst[((c * NDB + db) * 16 + r) * 64] = oacc[c][db][r];
        dst[(QC * NDB * 16 + 2 * c) * 64] = m_run[c];
        dst[(QC * NDB * 16 + 2 * c + 1) * 64] = l_run[c];
      }
    }
    __syncthreads();
    if (kg > 0) return;  // group 0 finishes the rows
#pragma unroll
    for (int g = 1; g < KG; ++g) {
      const float* src = mrg + ((g - 1) * QW + qw) * NREG * 64 + lane;
#pragma unroll
      for (int c = 0; c < QC; ++c) {
        const float m_o = src[(QC * NDB * 16 + 2 * c) * 64];
        const float l_o = src[(QC * NDB * 16 + 2 * c + 1) * 64];
        const float m_new = fmaxf(m_run[c], m_o);
        const float m_ref = m_new == -INFINITY ? 0.f : m_new;  // both groups saw no key
        const float a_self = __builtin_amdgcn_exp2f(m_run[c] - m_ref);
        const float a_other = __builtin_amdgcn_exp2f(m_o - m_ref);
        m_run[c] = m_new;
        l_run[c] = l_run[c] * a_self + l_o * a_other;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            oacc[c][db][r] = oacc[c][db][r] * a_self + src[((c * NDB + db) * 16 + r) * 64] * a_other;
      }
    }
  }

  // ---- epilogue: O = O / l, LSE = (m + log2 l) ln 2 -----------------------
#pragma unroll
  for (int c = 0; c < QC; ++c) {
    const float lt = half_sum(l_run[c]);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const int qrow = qw0 + c * 32 + l32;
    if (qrow < lq) {
      float* op = obase + (int64_t)qrow * a.o_ss + hh * 4;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float4 w;
          w.x = oacc[c][db][4 * g + 0] * inv;
          w.y = oacc[c][db][4 * g + 1] * inv;
          w.z = oacc[c][db][4 * g + 2] * inv;
          w.w = oacc[c][db][4 * g + 3] * inv;
          *reinterpret_cast<float4*>(op + db * 32 + 8 * g) = w;
        }
      }
      if (a.lse != nullptr && hh == 0) {
        const float v = lt > 0.f ? (m_run[c] + __log2f(lt)) * kLn2 : -INFINITY;
        a.lse[lseoff + (int64_t)h * a.lse_hs + qrow] = v;
      }
    }
  }
}

// ----------------------------------------------------------------------------
// Ping-pong variant: 8 waves, two groups of four (one wave of each group per
// SIMD).  Each wave owns 32 queries and alternates two phases, separated by
// workgroup barriers, offset by one phase between the groups:
//   matrix phase:  O^T += V^T P^T for tile j-1, then S^T = K Q^T for tile j
//   vector phase:  mask, row max, (rare) rescale, exp2 and bf16 packing of
//                  tile j, plus this group's half of the staging: group 0
//                  writes K of tile j+1 to LDS, group 1 writes V^T of tile j+1
// so on every SIMD one wave keeps the matrix core busy while the other runs
// the softmax arithmetic.  Tile j lives in LDS buffer j mod 3; the phase
// offsets make every write land in a buffer no wave is reading.
template <int D, bool VARLEN>
__global__ __launch_bounds__(512, 2) void attn_fwd_pingpong_kernel(const AttnArgs a) {
  constexpr int WAVES = 8;
  constexpr int BN = 64;
  constexpr int BM = WAVES * 32;
  constexpr int NBUF = 3;
  constexpr int GT = 256;                 // threads per group
  constexpr int KS = D + 8;
  constexpr int VS = BN + 8;
  constexpr int KT_ELEMS = BN * KS;
  constexpr int VT_ELEMS = D * VS;
  constexpr int NKB = BN / 32;
  constexpr int NDS = D / 16;
  constexpr int NDB = D / 32;
  constexpr int K_UNITS = BN * D / 8;
  constexpr int K_PER = (K_UNITS + GT - 1) / GT;
  constexpr int V_UNITS = (BN / 4) * (D / 8);
  constexpr int V_PER = (V_UNITS + GT - 1) / GT;

  __shared__ __attribute__((aligned(16))) uint16_t ks[NBUF * KT_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t vt[NBUF * VT_ELEMS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;
  const int gtid = tid & (GT - 1);
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  const int rows = a.nseq * a.hq;
  const int id = blockIdx.x;
  const int qb_rev = id / rows;
  int p = id - qb_rev * rows;
  if (a.xcd_remap) p = (p & 7) * (rows >> 3) + (p >> 3);
  const int seq = p / a.hq;
  const int h = p - seq * a.hq;
  const int qb = a.causal ? (a.n_qb - 1 - qb_rev) : qb_rev;
  int lq, lk;
  int64_t qoff, koff, voff, ooff, lseoff;
  if constexpr (VARLEN) {
    const SeqRows sr = seq_rows(a, seq);
    lq = sr.lq;
    lk = sr.lk;
    qoff = (int64_t)sr.q_row * a.q_ss;
    koff = (int64_t)sr.k_row * a.k_ss;
    voff = (int64_t)sr.k_row * a.v_ss;
    ooff = (int64_t)sr.q_row * a.o_ss;
    lseoff = sr.qs;
  } else {
    lq = a.sq;
    lk = a.sk;
    qoff = (int64_t)seq * a.q_bs;
    koff = (int64_t)seq * a.k_bs;
    voff = (int64_t)seq * a.v_bs;
    ooff = (int64_t)seq * a.o_bs;
    lseoff = (int64_t)seq * a.lse_bs;
  }
  const int q0 = qb * BM;
  if (q0 >= lq) return;
  const int kvh = h / a.group;
  const uint16_t* qbase = a.q + qoff + (int64_t)h * a.q_hs;
  const uint16_t* kbase = a.k + koff + (int64_t)kvh * a.k_hs;
  const uint16_t* vbase = a.v + voff + (int64_t)kvh * a.v_hs;
  float* obase = a.o + ooff + (int64_t)h * a.o_hs;

  const int off = lk - lq;
  int kend = lk;
  if (a.causal) kend = min(lk, q0 + BM + off);
  const int n_kt = kend > 0 ? (kend + BN - 1) / BN : 0;
  const int qw0 = q0 + wave * 32;
  int kend_w = lk;
  if (a.causal) kend_w = min(lk, qw0 + 32 + off);
  if (qw0 >= lq) kend_w = 0;
  const int nw = kend_w > 0 ? (kend_w + BN - 1) / BN : 0;

  const __amdgpu_buffer_rsrc_t qrs = make_rsrc(qbase, span_bytes(lq, a.q_ss));
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(kbase, span_bytes(lk, a.k_ss));
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vbase, span_bytes(lk, a.v_ss));
  const uint32_t k_row_bytes = (uint32_t)a.k_ss * 2;
  const uint32_t v_row_bytes = (uint32_t)a.v_ss * 2;
  u32x4 qraw[NDS];
  {
    const uint32_t qoff_b = (uint32_t)(qw0 + l32) * (uint32_t)a.q_ss * 2 + hh * 16;
#pragma unroll
    for (int s = 0; s < NDS; ++s)
      qraw[s] = __builtin_amdgcn_raw_buffer_load_b128(qrs, (int)(qoff_b + 32 * s), 0, 0);
  }
  bf16x8 qf[NDS];
#pragma unroll
  for (int s = 0; s < NDS; ++s) {
    asm volatile("" : "+v"(qraw[s]));
    qf[s] = __builtin_bit_cast(bf16x8, q_sign(qraw[s], a.q_xor, a.q_clear));
  }

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  // ---- staging: group 0 moves K tiles, group 1 moves V tiles ----------------
  uint4 kreg[K_PER];
  uint4 vreg[V_PER][4];
  auto k_fetch = [&](int kt) {
    const uint32_t kbeg = kt * BN;
#pragma unroll
    for (int i = 0; i < K_PER; ++i) {
      const int u = gtid + i * GT;
      if (K_UNITS % GT == 0 || u < K_UNITS) {
        const uint32_t row = u / (D / 8);
        const uint32_t col = (u % (D / 8)) * 16;
        kreg[i] = buf_ld16(krs, (kbeg + row) * k_row_bytes + col);
      }
    }
  };
  auto k_stage = [&](int buf) {
#pragma unroll
    for (int i = 0; i < K_PER; ++i) {
      const int u = gtid + i * GT;
      if (K_UNITS % GT == 0 || u < K_UNITS) {
        const int row = u / (D / 8);
        const int col = (u % (D / 8)) * 8;
        *reinterpret_cast<uint4*>(ks + buf * KT_ELEMS + row * KS + col) = kreg[i];
      }
    }
  };
  auto v_fetch = [&](int kt) {
    const uint32_t kbeg = kt * BN;
#pragma unroll
    for (int i = 0; i < V_PER; ++i) {
      const int u = gtid + i * GT;
      if (V_UNITS % GT == 0 || u < V_UNITS) {
        const uint32_t kq = u % (BN / 4);
        const uint32_t dq = u / (BN / 4);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          vreg[i][j] = buf_ld16(vrs, (kbeg + kq * 4 + j) * v_row_bytes + dq * 16);
      }
    }
  };
  auto v_stage = [&](int buf) {
#pragma unroll
    for (int i = 0; i < V_PER; ++i) {
      const int u = gtid + i * GT;
      if (V_UNITS % GT == 0 || u < V_UNITS) {
        const int kq = u % (BN / 4);
        const int dq = u / (BN / 4);
        const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&vreg[i][0]);
        const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&vreg[i][1]);
        const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&vreg[i][2]);
        const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&vreg[i][3]);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
          uint2 out;
          out.x = __builtin_amdgcn_perm(w1[e >> 1], w0[e >> 1], sel);
          out.y = __builtin_amdgcn_perm(w3[e >> 1], w2[e >> 1], sel);
          *reinterpret_cast<uint2*>(vt + buf * VT_ELEMS + (dq * 8 + e) * VS + kq * 4) = out;
        }
      }
    }
  };

  const uint16_t* k_lane = ks + key_of_row(l32) * KS + hh * 8;
  const uint16_t* v_lane = vt + l32 * VS + hh * 8;
  f32x16 sacc[NKB];
  bf16x8 pf[NKB][2];

  // ---- prologue: tile 0 staged by everyone; tile 1 fetched by its group ------
  if (n_kt > 0) {
    if (grp == 0) { k_fetch(0); k_stage(0); } else { v_fetch(0); v_stage(0); }
  }
  if (n_kt > 1) {
    if (grp == 0) k_fetch(1); else v_fetch(1);
  }
  __syncthreads();

  const int n_phase = 2 * n_kt + 2;
  for (int t = 0; t < n_phase; ++t) {
    const int my = t - grp;
    if (my >= 0) {
      const int j = my >> 1;
      if ((my & 1) == 0) {
        // ---- matrix phase: PV of tile j-1, QK of tile j -------------------------
        __builtin_amdgcn_s_setprio(1);
        const bool do_pv = j >= 1 && j - 1 < nw;
        const bool do_qk = j < nw;
        const uint16_t* vd = v_lane + ((j + NBUF - 1) % NBUF) * VT_ELEMS;
        const uint16_t* kd = k_lane + (j % NBUF) * KT_ELEMS;
        auto pv_block = [&]() {
#pragma unroll
          for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
              for (int tt = 0; tt < 2; ++tt) {
                const bf16x8 vf =
                    *reinterpret_cast<const bf16x8*>(vd + db * 32 * VS + kb * 32 + 16 * tt);
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[kb][tt], oacc[db], 0, 0, 0);
              }
        };
        auto qk_block = [&]() {
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int s = 0; s < NDS; ++s) {
              const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kd + kb * 32 * KS + 16 * s);
              sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s],
                                                                 s == 0 ? f32x16{} : sacc[kb], 0, 0, 0);
            }
        };
        if (do_pv && do_qk) {
          // one straight-line block; keep kLdsAhead fragment reads in flight
          pv_block();
          qk_block();
          lds_pipeline_hint<NDB * NKB * 2 + NKB * NDS>();
        } else if (do_pv) {
          pv_block();
        } else if (do_qk) {
          qk_block();
        }
        __builtin_amdgcn_s_setprio(0);
      } else {
        // ---- vector phase: softmax of tile j, staging of tile j+1 ---------------
        if (j < nw) {
          const int kbeg = j * BN;
          if ((kbeg + BN > lk) || (a.causal && kbeg + BN - 1 > qw0 + off)) {
            keep_branch();
            const int lim = a.causal ? min(lk - 1, qw0 + l32 + off) : lk - 1;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) mask_block(sacc[kb], lim - kbeg - kb * 32 - hh * 8);
          }
          float mx0 = -INFINITY, mx1 = -INFINITY;
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
              mx0 = fmaxf(mx0, sacc[kb][r]);
              mx1 = fmaxf(mx1, sacc[kb][r + 1]);
            }
          const float mx = half_max(fmaxf(mx0, mx1));
          const float cand = mx * a.c;
          const bool grow = cand > m_run + kRescaleThreshold;
          if (__builtin_amdgcn_ballot_w64(grow) != 0) {
            const float m_new = grow ? cand : m_run;
            const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
          }
          const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
          float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const float pv = __builtin_amdgcn_exp2f(fmaf(sacc[kb][r], a.c, -m_use));
              sacc[kb][r] = pv;
              if (r & 1) rs1 += pv; else rs0 += pv;
            }
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
              uint4 u;
              u.x = pack_bf16x2(sacc[kb][8 * tt + 0], sacc[kb][8 * tt + 1]);
              u.y = pack_bf16x2(sacc[kb][8 * tt + 2], sacc[kb][8 * tt + 3]);
              u.z = pack_bf16x2(sacc[kb][8 * tt + 4], sacc[kb][8 * tt + 5]);
              u.w = pack_bf16x2(sacc[kb][8 * tt + 6], sacc[kb][8 * tt + 7]);
              pf[kb][tt] = as_bf16x8(u);
            }
          }
          l_run += rs0 + rs1;
        }
        if (j + 1 < n_kt) {
          if (grp == 0) {
            k_stage((j + 1) % NBUF);
            if (j + 2 < n_kt) k_fetch(j + 2);
          } else {
            v_stage((j + 1) % NBUF);
            if (j + 2 < n_kt) v_fetch(j + 2);
          }
        }
      }
    }
    __syncthreads();
  }

  const float lt = half_sum(l_run);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  const int qrow = qw0 + l32;
  if (qrow < lq) {
    float* op = obase + (int64_t)qrow * a.o_ss + hh * 4;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float4 w;
        w.x = oacc[db][4 * g + 0] * inv;
        w.y = oacc[db][4 * g + 1] * inv;
        w.z = oacc[db][4 * g + 2] * inv;
        w.w = oacc[db][4 * g + 3] * inv;
        *reinterpret_cast<float4*>(op + db * 32 + 8 * g) = w;
      }
    if (a.lse != nullptr && hh == 0)
      a.lse[lseoff + (int64_t)h * a.lse_hs + qrow] =
          lt > 0.f ? (m_run + __log2f(lt)) * kLn2 : -INFINITY;
  }
}

// ----------------------------------------------------------------------------
// DMA-staged variant.
//
// K and V tiles go from HBM straight into LDS with buffer_load ... lds (each
// lane's 16 bytes land at LDS base + 16 x lane, so a wave instruction fills 1
// KiB of LDS; the global address of every lane is free).  No staging
// registers, no staging VALU work, and loads can run two tiles ahead.
//  * Rows are stored unpadded; 16-byte chunks are XOR-swizzled per row so the
//    two read patterns stay conflict-free: the K fragment read (16 lanes, 16
//    different rows, one chunk each) and the transposed V read (half a wave,
//    4 rows x 4 chunks).
//  * V stays row-major; the A operand of O^T += V^T P^T comes from two
//    ds_read_b64_tr_b16 per MFMA: within each 16-lane group that instruction
//    gives lane i element (i mod 4) of the 8-byte chunks addressed by lanes
//    4e + i/4 (e = 0..3), so each lane addresses 4 dims of one key row and
//    receives 4 keys of one dim.
//  * NBUF tile buffers are separate LDS objects and the key loop is unrolled
//    by NBUF, so the compiler can tell the buffer being read from the one the
//    DMA is filling; an explicit vmcnt wait before each barrier publishes the
//    next tile.

template <int D>
__device__ __forceinline__ int swz_k(int row) {
  if constexpr (D >= 128) return row & 15;
  else if constexpr (D == 64) return (row >> 1) & 7;
  else return (row >> 2) & 3;
}
template <int D>
__device__ __forceinline__ int swz_v(int row) {
  if constexpr (D >= 128) return (row & 3) << 2;
  else if constexpr (D == 64) return ((row >> 1) & 1) << 2;
  else return 0;
}

template <int D, int WAVES, int KG, int NBUF, bool VARLEN, int SUB = 1, int WIDE = 0>
__global__ __launch_bounds__(WAVES * 64, D == 256 ? 1 : 2) void attn_fwd_dma_kernel(const AttnArgs a) {
  constexpr int NT = WAVES * 64;
  constexpr int BN0 = WIDE ? 128 : (D == 256 || KG == 4) ? 32 : 64;  // keys per compute sub-tile
  constexpr int BN = SUB * BN0;              // keys per DMA tile (one barrier each)
  constexpr int QW = WAVES / KG;
  constexpr int BM = QW * 32;
  constexpr int CPR = D / 8;                 // 16-byte chunks per row
  constexpr int TILE = BN * D;               // elements of one K (or V) tile
  constexpr int IPT = BN * CPR / 64;         // 1 KiB DMA instructions per tile
  constexpr int NK = KG * IPT;               // ... for the K tiles of one step (same for V)
  static_assert(NK % WAVES == 0, "DMA instructions must split evenly over the waves");
  constexpr int PER_WAVE = 2 * NK / WAVES;   // DMA instructions one wave issues per step
  constexpr int NKB = BN0 / 32;
  constexpr int NDS = D / 16;
  constexpr int NDB = D / 32;
  static_assert(NBUF == 2 || NBUF == 3, "two or three buffers");

  __shared__ __attribute__((aligned(16))) uint16_t ks0[KG * TILE], vs0[KG * TILE];
  __shared__ __attribute__((aligned(16))) uint16_t ks1[KG * TILE], vs1[KG * TILE];
  __shared__ __attribute__((aligned(16))) uint16_t ks2[NBUF > 2 ? KG * TILE : 8];
  __shared__ __attribute__((aligned(16))) uint16_t vs2[NBUF > 2 ? KG * TILE : 8];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kg = wave / QW;
  const int qw = wave - kg * QW;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  const int id = blockIdx.x;
  int seq, h, qb_rev, part;
  if (a.xcd_remap == 2) {
    // sequence-major: all blocks of one sequence (longest first), its heads
    // spread so each XCD keeps hq/8 fixed heads and their K/V in its L2
    const int per_level = a.n_split * a.hq;
    const int per_seq = a.n_qb * per_level;
    seq = id / per_seq;
    int r = id - seq * per_seq;
    qb_rev = r / per_level;
    r -= qb_rev * per_level;
    part = r / a.hq;
    const int j = r - part * a.hq;
    h = (j & 7) * (a.hq >> 3) + (j >> 3);
  } else if (VARLEN && a.xcd_remap == 4) {
    // compact: sequence s owns block slots [cu_q[s] / BM + s, ...), disjoint and
    // increasing in s; the workgroup finds its sequence by binary search.  The
    // heads of one slot are consecutive, so each XCD keeps hq/8 fixed heads.
    const int j = id % a.hq;
    h = (a.hq % 8 == 0) ? (j & 7) * (a.hq >> 3) + (j >> 3) : j;
    const int vb = id / a.hq;
    int lo = 0, hi = a.nseq - 1;  // the last sequence whose first slot is <= vb
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.cu_q[mid] / BM + mid <= vb) lo = mid;
      else hi = mid - 1;
    }
    seq = lo;
    qb_rev = vb - (a.cu_q[seq] / BM + seq);  // block slot within the sequence
    part = 0;
  } else if (a.xcd_remap == 3) {
    // (sequence, head) units dealt round-robin to the XCDs, all blocks of a
    // unit in a row on its XCD (no split parts in this order)
    const int local = id >> 3;
    const int u = local / a.n_qb;
    qb_rev = local - u * a.n_qb;
    const int p = u * 8 + (id & 7);
    if (p >= a.nseq * a.hq) return;
    seq = p / a.hq;
    h = p - seq * a.hq;
    part = 0;
  } else {
    const int rows = a.nseq * a.hq;
    const int per_qb = rows * a.n_split;
    qb_rev = id / per_qb;
    const int rem = id - qb_rev * per_qb;
    part = rem / rows;
    int p = rem - part * rows;
    if (a.xcd_remap) p = (p & 7) * (rows >> 3) + (p >> 3);
    seq = p / a.hq;
    h = p - seq * a.hq;
  }
  int qb = a.causal ? (a.n_qb - 1 - qb_rev) : qb_rev;
  int lq, lk;
  int64_t qoff, koff, voff, ooff, lseoff;
  if constexpr (VARLEN) {
    const SeqRows sr = seq_rows(a, seq);
    lq = sr.lq;
    lk = sr.lk;
    if (a.xcd_remap == 4) {
      // slot qb_rev of this sequence's blocks, longest first when causal
      const int nb = (lq + BM - 1) / BM;
      if (qb_rev >= nb) return;
      qb = a.causal ? nb - 1 - qb_rev : qb_rev;
    }
    qoff = (int64_t)sr.q_row * a.q_ss;
    koff = (int64_t)sr.k_row * a.k_ss;
    voff = (int64_t)sr.k_row * a.v_ss;
    ooff = (int64_t)sr.q_row * a.o_ss;
    lseoff = sr.qs;
  } else {
    lq = a.sq;
    lk = a.sk;
    qoff = (int64_t)seq * a.q_bs;
    koff = (int64_t)seq * a.k_bs;
    voff = (int64_t)seq * a.v_bs;
    ooff = (int64_t)seq * a.o_bs;
    lseoff = (int64_t)seq * a.lse_bs;
  }
  const int q0 = qb * BM;
  if (q0 >= lq) return;
  const int kvh = h / a.group;
  const uint16_t* qbase = a.q + qoff + (int64_t)h * a.q_hs;
  const uint16_t* kbase = a.k + koff + (int64_t)kvh * a.k_hs;
  const uint16_t* vbase = a.v + voff + (int64_t)kvh * a.v_hs;
  float* obase = a.o + ooff + (int64_t)h * a.o_hs;

  const int off = lk - lq;
  int kend = lk;
  if (a.causal) kend = min(lk, q0 + BM + off);
  const int n_kt_all = kend > 0 ? (kend + BN - 1) / BN : 0;
  // key tiles [t_begin, t_end) of this part of the block
  const int n_parts = split_parts(n_kt_all, a.n_split, a.split_tiles);
  if (part >= n_parts) return;
  const int per_part = (n_kt_all + n_parts - 1) / n_parts;
  const int t_begin = part * per_part;
  const int t_end = min(n_kt_all, t_begin + per_part);
  const int n_kt = max(t_end - t_begin, 0);
  const int n_steps = (n_kt + KG - 1) / KG;
  const int qw0 = q0 + qw * 32;
  int kend_w = lk;
  if (a.causal) kend_w = min(lk, qw0 + 32 + off);
  if (qw0 >= lq) kend_w = 0;

  const __amdgpu_buffer_rsrc_t qrs = make_rsrc(qbase, span_bytes(lq, a.q_ss));
  const uint32_t k_row_bytes = (uint32_t)a.k_ss * 2;
  const uint32_t v_row_bytes = (uint32_t)a.v_ss * 2;
  const u32x4 kdesc = make_desc(kbase, span_bytes(lk, a.k_ss));
  const u32x4 vdesc = make_desc(vbase, span_bytes(lk, a.v_ss));

  u32x4 qraw[NDS];
  {
    const uint32_t qoff_b = (uint32_t)(qw0 + l32) * (uint32_t)a.q_ss * 2 + hh * 16;
#pragma unroll
    for (int s = 0; s < NDS; ++s)
      qraw[s] = __builtin_amdgcn_raw_buffer_load_b128(qrs, (int)(qoff_b + 32 * s), 0, 0);
  }
  bf16x8 qf[NDS];
#pragma unroll
  for (int s = 0; s < NDS; ++s) {
    asm volatile("" : "+v"(qraw[s]));
    qf[s] = __builtin_bit_cast(bf16x8, q_sign(qraw[s], a.q_xor, a.q_clear));
  }

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  // ---- DMA of one step (KG tiles of K and of V) into buffer B ----------------
  // Byte offsets of this wave's DMA instructions within a step's tiles (the
  // same every step): pair i is the wave's i-th K and V instruction.  The
  // step's first key moves the buffer base instead (scalar arithmetic), so an
  // instruction is one M0 write and one load, with no vector work.
  constexpr int NP = NK / WAVES;
  uint32_t koffp[NP], voffp[NP];
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int ins = wave * NP + i;  // 0 .. NK-1, wave-uniform
    const int g = ins / IPT;
    const int cgi = ins - g * IPT;
    const int slot = cgi * 64 + lane;
    const int row = slot / CPR;      // row within the tile
    const int phys = slot - row * CPR;
    koffp[i] = (uint32_t)(g * BN + row) * k_row_bytes + (uint32_t)((phys ^ swz_k<D>(row)) * 16);
    voffp[i] = (uint32_t)(g * BN + row) * v_row_bytes + (uint32_t)((phys ^ swz_v<D>(row)) * 16);
  }
  // the buffer of rows [first row of the step, end of sequence)
  struct StepDesc {
    u32x4 k, v;
  };
  auto descs_of = [&](int step) __attribute__((always_inline)) {
    const uint32_t kbeg = __builtin_amdgcn_readfirstlane((t_begin + step * KG) * BN);
    return StepDesc{desc_advance(kdesc, kbeg * k_row_bytes), desc_advance(vdesc, kbeg * v_row_bytes)};
  };
  auto dma_pair = [&](auto Bc, const StepDesc& sd, int i) __attribute__((always_inline)) {
    constexpr int B = decltype(Bc)::value;
    uint16_t* kd = B == 0 ? ks0 : B == 1 ? ks1 : ks2;
    uint16_t* vd = B == 0 ? vs0 : B == 1 ? vs1 : vs2;
    const int ins = wave * NP + i;
    const int g = ins / IPT;
    const int cgi = ins - g * IPT;
    dma16(sd.k, koffp[i], __builtin_amdgcn_readfirstlane(lds_addr(kd + g * TILE + cgi * 512)));
    dma16(sd.v, voffp[i], __builtin_amdgcn_readfirstlane(lds_addr(vd + g * TILE + cgi * 512)));
  };
  auto dma = [&](auto Bc, int step) {
    const StepDesc sd = descs_of(step);
#pragma unroll
    for (int i = 0; i < NP; ++i) dma_pair(Bc, sd, i);
  };
  // lane-constant parts of the fragment addresses
  int krow[NKB];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) krow[kb] = (kb * 32 + key_of_row(l32)) * D;
  const int ksw = swz_k<D>(key_of_row(l32));
  const int vrow0 = 8 * hh + ((lane & 15) >> 2);
  const int vsw = swz_v<D>(vrow0);
  const int vcc = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);  // chunk within a 32-dim block
  const int vhalf = (lane & 1) * 4;

  // one sub-tile of BN0 keys starting at key kbeg, rows kd / vd of the tile
  auto sub_tile = [&](const uint16_t* kd, const uint16_t* vd, int kbeg) __attribute__((always_inline)) {
    if (kbeg >= kend_w) return;
    f32x16 sacc[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int s = 0; s < NDS; ++s) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kd + krow[kb] + (((2 * s + hh) ^ ksw) * 8));
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], s == 0 ? f32x16{} : sacc[kb],
                                                           0, 0, 0);
      }
    lds_pipeline_hint<NKB * NDS>();
    if ((kbeg + BN0 > lk) || (a.causal && kbeg + BN0 - 1 > qw0 + off)) {
      keep_branch();
      const int lim = a.causal ? min(lk - 1, qw0 + l32 + off) : lk - 1;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) mask_block(sacc[kb], lim - kbeg - kb * 32 - hh * 8);
    }
    float mx0 = -INFINITY, mx1 = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        mx0 = fmaxf(mx0, sacc[kb][r]);
        mx1 = fmaxf(mx1, sacc[kb][r + 1]);
      }
    const float cand = half_max(fmaxf(mx0, mx1)) * a.c;
    const bool grow = cand > m_run + kRescaleThreshold;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float m_new = grow ? cand : m_run;
      const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
    }
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
    bf16x8 pf[NKB][2];
    float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pvl = __builtin_amdgcn_exp2f(fmaf(sacc[kb][r], a.c, -m_use));
        sacc[kb][r] = pvl;
        if (r & 1) rs1 += pvl; else rs0 += pvl;
      }
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        uint4 u;
        u.x = pack_bf16x2(sacc[kb][8 * t + 0], sacc[kb][8 * t + 1]);
        u.y = pack_bf16x2(sacc[kb][8 * t + 2], sacc[kb][8 * t + 3]);
        u.z = pack_bf16x2(sacc[kb][8 * t + 4], sacc[kb][8 * t + 5]);
        u.w = pack_bf16x2(sacc[kb][8 * t + 6], sacc[kb][8 * t + 7]);
        pf[kb][t] = as_bf16x8(u);
      }
    }
    l_run += rs0 + rs1;
    // Key-block-major order: the products of the first 32 keys need only
    // their own probabilities, so they can start while the exponentials of
    // the second 32 keys are still being computed (measured 3-5 % faster
    // than accumulator-major order at head_dim 128).
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          // rows kb*32 + 16t + 8hh + (lane%16)/4 (+4 for the second read)
          const uint16_t* src = vd + (kb * 32 + 16 * t + vrow0) * D + (((db * 4) ^ vsw) + vcc) * 8 + vhalf;
          const uint2 lo = ds_read_tr16(src);
          const uint2 hi = ds_read_tr16(src + 4 * D);
          const bf16x8 vf = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[kb][t], oacc[db], 0, 0, 0);
        }
  };

  auto compute = [&](auto Bc, int step) {
    constexpr int B = decltype(Bc)::value;
    const uint16_t* kd = (B == 0 ? ks0 : B == 1 ? ks1 : ks2) + kg * TILE;
    const uint16_t* vd = (B == 0 ? vs0 : B == 1 ? vs1 : vs2) + kg * TILE;
    const int kt = t_begin + step * KG + kg;
    if (kt >= t_end) return;
#pragma unroll
    for (int sb = 0; sb < SUB; ++sb) sub_tile(kd + sb * BN0 * D, vd + sb * BN0 * D, kt * BN + sb * BN0);
  };

  // ---- pipeline: step s reads buffer s % NBUF; the DMA runs NBUF-1 steps ahead --
  if (n_steps > 0) dma(std::integral_constant<int, 0>{}, 0);
  if constexpr (NBUF == 3) {
    if (n_steps > 1) {
      dma(std::integral_constant<int, 1>{}, 1);
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(PER_WAVE));
    } else {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    }
  } else {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  }
  __syncthreads();

  auto iteration = [&](auto Bc, int step) {
    constexpr int B = decltype(Bc)::value;
    constexpr int BA = (B + NBUF - 1) % NBUF;  // buffer the DMA ahead fills
    const bool ahead = step + NBUF - 1 < n_steps;
    if (ahead) dma(std::integral_constant<int, BA>{}, step + NBUF - 1);
    compute(Bc, step);
    // publish step+1: its DMA must be complete; the one issued above may run on
    if (NBUF == 3 && ahead) __builtin_amdgcn_s_waitcnt(vmcnt_imm(PER_WAVE));
    else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();
  };
  for (int step = 0; step < n_steps; step += NBUF) {
    iteration(std::integral_constant<int, 0>{}, step);
    if (step + 1 < n_steps) iteration(std::integral_constant<int, 1>{}, step + 1);
    if constexpr (NBUF == 3) {
      if (step + 2 < n_steps) iteration(std::integral_constant<int, 2>{}, step + 2);
    }
  }

  // ---- key-group merge (KG > 1): partial (m, l, O) through LDS ------------------
  // Sliced merge (the 32-dim blocks divide evenly over the groups): every
  // wave publishes its (m, l) and the O blocks of the other groups' dim
  // slices, one barrier, then each wave combines its own slice of the output
  // dims from all KG groups and stores just that slice.  The merge and the
  // stores of a block are then spread over all of its waves, behind a single
  // barrier.  The groups are combined in group order in every wave, so the
  // row sum (and thus the normaliser of every slice) is the same in all.
  constexpr bool SLICED = KG > 1 && NDB % KG == 0;
  constexpr int DSL = SLICED ? NDB / KG : NDB;  // 32-dim blocks this wave stores
  const int db0 = SLICED ? kg * DSL : 0;
  if constexpr (SLICED) {
    constexpr int NOUT = (NDB - DSL) * 16;  // O values a wave hands to the other groups, per lane
    constexpr int SLOT = NOUT + 2;          // plus m and l
    static_assert(2 * SLOT * 64 * 4 <= KG * TILE * 2, "two waves' partials per tile array");
    static_assert(WAVES == 8, "slots: two waves per tile array");
    auto slot_of = [&](int w) {
      uint16_t* s16 = (w >> 1) == 0 ? ks0 : (w >> 1) == 1 ? vs0 : (w >> 1) == 2 ? ks1 : vs1;
      return reinterpret_cast<float*>(s16) + (w & 1) * SLOT * 64 + lane;  // [reg][lane]
    };
    {
      float* my = slot_of(wave);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        if (db >= db0 && db < db0 + DSL) continue;
        const int j = db < db0 ? db : db - DSL;
#pragma unroll
        for (int r = 0; r < 16; ++r) my[(j * 16 + r) * 64] = oacc[db][r];
      }
      my[NOUT * 64] = m_run;
      my[(NOUT + 1) * 64] = l_run;
    }
    __syncthreads();
    float m_g[KG], l_g[KG];
#pragma unroll
    for (int g = 0; g < KG; ++g) {
      if (g == kg) {
        m_g[g] = m_run;
        l_g[g] = l_run;
      } else {
        const float* o = slot_of(g * QW + qw);
        m_g[g] = o[NOUT * 64];
        l_g[g] = o[(NOUT + 1) * 64];
      }
    }
    float m_all = m_g[0];
#pragma unroll
    for (int g = 1; g < KG; ++g) m_all = fmaxf(m_all, m_g[g]);
    const float m_ref = m_all == -INFINITY ? 0.f : m_all;
    float al[KG];
    float l_tot = 0.f;
#pragma unroll
    for (int g = 0; g < KG; ++g) {
      al[g] = __builtin_amdgcn_exp2f(m_g[g] - m_ref);
      l_tot += l_g[g] * al[g];
    }
    f32x16 acc[DSL];
#pragma unroll
    for (int d = 0; d < DSL; ++d) acc[d] = f32x16{};
#pragma unroll
    for (int g = 0; g < KG; ++g) {
      const float* o = slot_of(g * QW + qw);
      const int gdb0 = g * DSL;  // group g's slice; where our blocks sit in its slot
#pragma unroll
      for (int d = 0; d < DSL; ++d) {
        if (g == kg) {
          // own blocks db0 + d: still in registers (db0 is wave-uniform)
#pragma unroll
          for (int db = 0; db < NDB; ++db)
            if (db == db0 + d) acc[d] += oacc[db] * al[g];
        } else {
          const int db = db0 + d;
          const int j = db < gdb0 ? db : db - DSL;
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[d][r] += o[(j * 16 + r) * 64] * al[g];
        }
      }
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int d = 0; d < DSL; ++d)
        if (db == d) oacc[db] = acc[d];  // this wave's slice now sits in oacc[0..DSL)
    m_run = m_all;
    l_run = l_tot;
  } else if constexpr (KG > 1) {
    static_assert(KG == 2 || KG == 4, "merge written for two or four key groups");
    constexpr int NREG = NDB * 16 + 2;
    static_assert(NREG * 64 * 4 <= KG * TILE * 2, "one wave's partial must fit one tile array");
    static_assert(QW * (KG / 2) <= 4, "merge slots: ks0, vs0, ks1, vs1");
    auto slot_of = [&](int i) {
      uint16_t* s16 = i == 0 ? ks0 : i == 1 ? vs0 : i == 2 ? ks1 : vs1;
      return reinterpret_cast<float*>(s16) + lane;  // [reg][lane]
    };
    auto put = [&](float* slot) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) slot[(db * 16 + r) * 64] = oacc[db][r];
      slot[(NDB * 16) * 64] = m_run;
      slot[(NDB * 16 + 1) * 64] = l_run;
    };
    auto take = [&](const float* slot) {
      const float m_o = slot[(NDB * 16) * 64];
      const float l_o = slot[(NDB * 16 + 1) * 64];
      const float m_new = fmaxf(m_run, m_o);
      const float m_ref = m_new == -INFINITY ? 0.f : m_new;
      const float a_self = __builtin_amdgcn_exp2f(m_run - m_ref);
      const float a_other = __builtin_amdgcn_exp2f(m_o - m_ref);
      m_run = m_new;
      l_run = l_run * a_self + l_o * a_other;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          oacc[db][r] = oacc[db][r] * a_self + slot[(db * 16 + r) * 64] * a_other;
    };
    if constexpr (KG == 4) {
      // groups 2 and 3 hand their partials to groups 0 and 1
      if (kg >= 2) put(slot_of((kg - 2) * QW + qw));
      __syncthreads();
      if (kg >= 2) return;
      take(slot_of(kg * QW + qw));
      // then group 1 to group 0, through the slot group 1 has just read
      if (kg == 1) put(slot_of(QW + qw));
      __syncthreads();
      if (kg == 1) return;
      take(slot_of(QW + qw));
    } else {
      if (kg == 1) put(slot_of(qw));
      __syncthreads();
      if (kg == 1) return;
      take(slot_of(qw));
    }
  }

  const float lt = half_sum(l_run);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  const int qrow = qw0 + l32;
  if (n_parts > 1) {
    // partial result of this part: O / l and the base-2 LSE, merged later
    if (qrow < lq) {
      const int64_t slot = (((int64_t)(seq * a.hq + h) * a.n_qb + qb) * a.n_split + part) * BM +
                           (qrow - q0);
      float* op = a.part_o + slot * D + hh * 4 + db0 * 32;
#pragma unroll
      for (int db = 0; db < DSL; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float4 w;
          w.x = oacc[db][4 * g + 0] * inv;
          w.y = oacc[db][4 * g + 1] * inv;
          w.z = oacc[db][4 * g + 2] * inv;
          w.w = oacc[db][4 * g + 3] * inv;
          *reinterpret_cast<float4*>(op + db * 32 + 8 * g) = w;
        }
      if (hh == 0 && kg == 0) a.part_lse[slot] = lt > 0.f ? m_run + __log2f(lt) : -INFINITY;
    }
    return;
  }
  if (qrow < lq) {
    float* op = obase + (int64_t)qrow * a.o_ss + hh * 4 + db0 * 32;
#pragma unroll
    for (int db = 0; db < DSL; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float4 w;
        w.x = oacc[db][4 * g + 0] * inv;
        w.y = oacc[db][4 * g + 1] * inv;
        w.z = oacc[db][4 * g + 2] * inv;
        w.w = oacc[db][4 * g + 3] * inv;
        *reinterpret_cast<float4*>(op + db * 32 + 8 * g) = w;
      }
    if (a.lse != nullptr && hh == 0 && kg == 0)
      a.lse[lseoff + (int64_t)h * a.lse_hs + qrow] =
          lt > 0.f ? (m_run + __log2f(lt)) * kLn2 : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// Merge of split query blocks.  Part r of a block holds O_r (normalised by its
// own row sum) and L_r = log2 of that row sum in base-2 exponent units; the
// whole block is O = sum_r 2^(L_r - L) O_r with L = log2 sum_r 2^(L_r), the
// log-sum-exp rule that combines softmax partials over disjoint key ranges
// ("Intro to FlashAttention on Ascend CANN", the running maximum and sum of
// the online softmax applied to whole parts).
// ---------------------------------------------------------------------------
// One thread per 4 output values; a workgroup covers kMergeRows rows of a
// block, so each thread waits on one round of loads only.
constexpr int kMergeRows = 8;

template <int D, bool VARLEN>
__global__ __launch_bounds__(kMergeRows * D / 4) void merge_split_kernel(const AttnArgs a, int bm) {
  const int rows = a.nseq * a.hq;
  const int chunks = bm / kMergeRows;
  const int blk = blockIdx.x / chunks;
  const int chunk = blockIdx.x - blk * chunks;
  const int qb = blk / rows;
  const int pr = blk - qb * rows;
  const int seq = pr / a.hq;
  const int h = pr - seq * a.hq;
  int lq, lk;
  int64_t ooff, lseoff;
  if constexpr (VARLEN) {
    const SeqRows sr = seq_rows(a, seq);
    lq = sr.lq;
    lk = sr.lk;
    ooff = (int64_t)sr.q_row * a.o_ss;
    lseoff = sr.qs;
  } else {
    lq = a.sq;
    lk = a.sk;
    ooff = (int64_t)seq * a.o_bs;
    lseoff = (int64_t)seq * a.lse_bs;
  }
  const int q0 = qb * bm;
  if (q0 >= lq) return;
  const int off = lk - lq;
  int kend = lk;
  if (a.causal) kend = min(lk, q0 + bm + off);
  const int n_kt = kend > 0 ? (kend + a.split_bn - 1) / a.split_bn : 0;
  const int np = split_parts(n_kt, a.n_split, a.split_tiles);
  if (np <= 1) return;  // the attention kernel wrote this block itself
  const int64_t base = ((int64_t)pr * a.n_qb + qb) * a.n_split * bm;
  constexpr int C4 = D / 4;
  {
    const int row = chunk * kMergeRows + (int)threadIdx.x / C4;
    const int c = (int)threadIdx.x % C4;
    if (q0 + row >= lq) return;
    float mx = -INFINITY;
    for (int r = 0; r < np; ++r) mx = fmaxf(mx, a.part_lse[base + (int64_t)r * bm + row]);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    float wsum = 0.f;
    if (mx != -INFINITY) {
      for (int r = 0; r < np; ++r) {
        const int64_t slot = base + (int64_t)r * bm + row;
        const float w = __builtin_amdgcn_exp2f(a.part_lse[slot] - mx);
        const float4 o = *reinterpret_cast<const float4*>(a.part_o + slot * D + 4 * c);
        acc.x = fmaf(w, o.x, acc.x);
        acc.y = fmaf(w, o.y, acc.y);
        acc.z = fmaf(w, o.z, acc.z);
        acc.w = fmaf(w, o.w, acc.w);
        wsum += w;
      }
      const float inv = 1.f / wsum;
      acc.x *= inv;
      acc.y *= inv;
      acc.z *= inv;
      acc.w *= inv;
    }
    float* op = a.o + ooff + (int64_t)(q0 + row) * a.o_ss + (int64_t)h * a.o_hs + 4 * c;
    *reinterpret_cast<float4*>(op) = acc;
    if (c == 0 && a.lse != nullptr)
      a.lse[lseoff + (int64_t)h * a.lse_hs + q0 + row] =
          mx == -INFINITY ? -INFINITY : (mx + __log2f(wsum)) * kLn2;
  }
}

// ---------------------------------------------------------------------------
// Software-pipelined kernel.
//
// Each wave overlaps its own work instead of relying on a second wave: while
// the matrix core computes the scores of tile j+1 (S_{j+1} = K_{j+1} Q^T), the
// VALU turns S_j into probabilities; then O += V_j^T P_j runs.  A barrier per
// tile keeps all waves of a workgroup in the same phase, so overlap between
// waves alone leaves the matrix core idle during the softmax; here it need not.
//
// Tiles arrive by LDS DMA into NBUF buffers; iteration j reads K of tile j+1
// and V of tile j and issues the DMA of tile j + NBUF - 1.
//
// LDS layout.  One DMA instruction moves 64 x 16 bytes = R = 64 / (D/8) rows
// of a tile.  Inside its 1 KiB the 16-byte chunk c of row-in-group i sits at
// slot c * R + (i ^ rot(c)) (chunk-major), and consecutive instructions are G
// bytes apart.  A fragment read then has the address (lane base) + (constant)
// for every K chunk pair and every V dim block, so the kernel needs only a
// handful of address registers, and the reads stay free of bank conflicts:
//  * K read: 16 consecutive lanes read one chunk of 16 consecutive rows; the
//    rows of one instruction are 16 bytes apart and G_K shifts the next
//    instruction by a quarter (D=128) or half (D=64) of 256 bytes.
//  * V transposed read: a 16-lane group reads 4 consecutive rows of two
//    adjacent chunks, 128 contiguous bytes for D=128; for D=64 rot() moves
//    one chunk of each pair (and of the 4-chunk set a 32-lane read covers) to
//    the other half of the bank range.
// K rows are stored in key_of_row order (the DMA lane picks the source row),
// so lane l reads row l and its scores come out in the order the P operand
// needs.
// ---------------------------------------------------------------------------
// (PipeLayout is defined in attn_device.h.)

template <int D, int BN, int WAVES, int NBUF, int MINW, bool VARLEN>
__global__ __launch_bounds__(WAVES * 64, MINW) void attn_fwd_pipe_kernel(const AttnArgs a) {
  using L = PipeLayout<D>;
  constexpr int BM = WAVES * 32;
  constexpr int R = L::R;
  constexpr int NI = BN / R;                  // DMA instructions per tile (K or V)
  static_assert(NI % WAVES == 0, "DMA instructions must split evenly over the waves");
  constexpr int NIW = NI / WAVES;             // ... per wave
  constexpr int PER_WAVE = 2 * NIW;           // vector-memory ops a wave issues per tile
  constexpr int KT = NI * L::GK;              // bytes of one K tile
  constexpr int VT = NI * L::GV;
  constexpr int NKB = BN / 32;
  constexpr int NDS = D / 16;
  constexpr int NDB = D / 32;
  static_assert(NBUF == 3 || NBUF == 4, "three or four buffers");

  __shared__ __attribute__((aligned(16))) unsigned char lds[NBUF * (KT + VT)];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  const int rows = a.nseq * a.hq;
  const int id = blockIdx.x;
  int qb_rev, p;
  if (a.xcd_remap == 3) {
    // (sequence, head) units dealt round-robin to the XCDs; all blocks of a
    // unit in a row on its XCD, so they read its K/V from that L2
    const int local = id >> 3;
    const int u = local / a.n_qb;
    qb_rev = local - u * a.n_qb;
    p = u * 8 + (id & 7);
    if (p >= rows) return;
  } else {
    qb_rev = id / rows;
    p = id - qb_rev * rows;
    if (a.xcd_remap) p = (p & 7) * (rows >> 3) + (p >> 3);
  }
  const int seq = p / a.hq;
  const int h = p - seq * a.hq;
  const int qb = a.causal ? (a.n_qb - 1 - qb_rev) : qb_rev;
  int lq, lk;
  int64_t qoff, koff, voff, ooff, lseoff;
  if constexpr (VARLEN) {
    const SeqRows sr = seq_rows(a, seq);
    lq = sr.lq;
    lk = sr.lk;
    qoff = (int64_t)sr.q_row * a.q_ss;
    koff = (int64_t)sr.k_row * a.k_ss;
    voff = (int64_t)sr.k_row * a.v_ss;
    ooff = (int64_t)sr.q_row * a.o_ss;
    lseoff = sr.qs;
  } else {
    lq = a.sq;
    lk = a.sk;
    qoff = (int64_t)seq * a.q_bs;
    koff = (int64_t)seq * a.k_bs;
    voff = (int64_t)seq * a.v_bs;
    ooff = (int64_t)seq * a.o_bs;
    lseoff = (int64_t)seq * a.lse_bs;
  }
  const int q0 = qb * BM;
  if (q0 >= lq) return;
  const int kvh = h / a.group;
  const uint16_t* qbase = a.q + qoff + (int64_t)h * a.q_hs;
  const uint16_t* kbase = a.k + koff + (int64_t)kvh * a.k_hs;
  const uint16_t* vbase = a.v + voff + (int64_t)kvh * a.v_hs;
  float* obase = a.o + ooff + (int64_t)h * a.o_hs;

  // Tiles of the block (every wave joins every DMA and barrier) and of this
  // wave: n_w tiles hold a key some query of the wave sees; the first n_full
  // of them are visible to all of its queries.
  const int off = lk - lq;
  int kend = lk;
  if (a.causal) kend = min(lk, q0 + BM + off);
  const int n_steps = kend > 0 ? (kend + BN - 1) / BN : 0;
  const int qw0 = q0 + wave * 32;
  int kend_w = lk;
  if (a.causal) kend_w = min(lk, qw0 + 32 + off);
  if (qw0 >= lq) kend_w = 0;
  const int n_w = kend_w > 0 ? (kend_w + BN - 1) / BN : 0;
  const int full_keys = a.causal ? min(lk, qw0 + off + 1) : lk;
  const int n_full = full_keys > 0 ? min(full_keys / BN, n_w) : 0;

  const __amdgpu_buffer_rsrc_t qrs = make_rsrc(qbase, span_bytes(lq, a.q_ss));
  const uint32_t k_row_bytes = (uint32_t)a.k_ss * 2;
  const uint32_t v_row_bytes = (uint32_t)a.v_ss * 2;
  const u32x4 kdesc = make_desc(kbase, span_bytes(lk, a.k_ss));
  const u32x4 vdesc = make_desc(vbase, span_bytes(lk, a.v_ss));

  u32x4 qraw[NDS];
  {
    const uint32_t qoff_b = (uint32_t)(qw0 + l32) * (uint32_t)a.q_ss * 2 + hh * 16;
#pragma unroll
    for (int s = 0; s < NDS; ++s)
      qraw[s] = __builtin_amdgcn_raw_buffer_load_b128(qrs, (int)(qoff_b + 32 * s), 0, 0);
  }
  bf16x8 qf[NDS];
#pragma unroll
  for (int s = 0; s < NDS; ++s) {
    asm volatile("" : "+v"(qraw[s]));
    qf[s] = __builtin_bit_cast(bf16x8, q_sign(qraw[s], a.q_xor, a.q_clear));
  }

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f, cand = -INFINITY;

  // ---- DMA: the lane's (row, chunk) in each of this wave's instructions ----
  uint32_t dk[NIW], dv[NIW];
#pragma unroll
  for (int i = 0; i < NIW; ++i) {
    const int q = wave * NIW + i;
    const int c = lane / R;
    const int row = q * R + ((lane % R) ^ L::rot(c));
    const int krow_src = (row & ~31) + key_of_row(row & 31);
    dk[i] = (uint32_t)krow_src * k_row_bytes + (uint32_t)c * 16;
    dv[i] = (uint32_t)row * v_row_bytes + (uint32_t)c * 16;
  }
  const uint32_t lds0 = lds_addr(lds);
  auto dma = [&](int t) {
    const int b = t % NBUF;
    const uint32_t kb_k = (uint32_t)t * BN * k_row_bytes;
    const uint32_t kb_v = (uint32_t)t * BN * v_row_bytes;
#pragma unroll
    for (int i = 0; i < NIW; ++i) {
      const int q = wave * NIW + i;
      dma16(kdesc, kb_k + dk[i], __builtin_amdgcn_readfirstlane(lds0 + b * KT + q * L::GK));
      dma16(vdesc, kb_v + dv[i], __builtin_amdgcn_readfirstlane(lds0 + NBUF * KT + b * VT + q * L::GV));
    }
  };

  // ---- fragment addresses: lane base + constant ------------------------------
  // K fragment (kb, s): row 32kb + l32, chunk 2s + hh.  V fragment (db, kb, t,
  // half): rows 32kb + 16t + 8hh + u (+4 for the second read), chunk 4db + vcc.
  const int u = (lane & 15) >> 2;
  const int vcc = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int kl[2] = {L::at(l32, hh, L::GK), L::at(l32, 2 + hh, L::GK)};
  const int vl[2] = {L::at(8 * hh + u, vcc, L::GV) + 8 * (lane & 1),
                     L::at(8 * hh + u + 4, vcc, L::GV) + 8 * (lane & 1)};
  auto kfrag = [&](uint32_t kt_base, int kb, int s) -> bf16x8 {
    // constant part: rows 32kb (32kb/R instructions), chunk pair s/2 (chunk 2s)
    const int cst = (32 * kb / R) * L::GK + 16 * R * 2 * (s & ~1);
    return *reinterpret_cast<const bf16x8*>(lds + kt_base + kl[s & 1] + cst);
  };
  auto vfrag = [&](uint32_t vt_base, int db, int kb, int t) -> bf16x8 {
    const int cst = ((32 * kb + 16 * t) / R) * L::GV + 16 * R * 4 * db;
    const uint2 lo = ds_read_tr16(reinterpret_cast<const uint16_t*>(lds + vt_base + vl[0] + cst));
    const uint2 hi = ds_read_tr16(reinterpret_cast<const uint16_t*>(lds + vt_base + vl[1] + cst));
    return as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
  };

  f32x16 S0[NKB], S1[NKB];

  auto qk = [&](int t, f32x16 (&S)[NKB]) {
    const uint32_t kt_base = (uint32_t)(t % NBUF) * KT;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int s = 0; s < NDS; ++s)
        S[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfrag(kt_base, kb, s), qf[s],
                                                        s == 0 ? f32x16{} : S[kb], 0, 0, 0);
  };

  auto mask = [&](f32x16 (&S)[NKB], int t) {
    keep_branch();
    const int kbeg = t * BN;
    const int lim = a.causal ? min(lk - 1, qw0 + l32 + off) : lk - 1;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) mask_block(S[kb], lim - kbeg - kb * 32 - hh * 8);
  };

  // row maximum in base-2 units; mx0/mx1 hold the running partial maxima
  auto rowmax_part = [&](const f32x16 (&S)[NKB], int e0, int ne, float& mx0, float& mx1) {
#pragma unroll
    for (int e = e0; e < e0 + ne; e += 2) {
      mx0 = fmaxf(mx0, S[e >> 4][e & 15]);
      mx1 = fmaxf(mx1, S[e >> 4][(e & 15) + 1]);
    }
  };
  auto rowmax = [&](const f32x16 (&S)[NKB]) {
    float mx0 = -INFINITY, mx1 = -INFINITY;
    rowmax_part(S, 0, NKB * 16, mx0, mx1);
    cand = half_max(fmaxf(mx0, mx1)) * a.c;
  };

  auto rescale = [&]() {
    const bool grow = cand > m_run + kRescaleThreshold;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float m_new = grow ? cand : m_run;
      const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
    }
  };

  // ---- one iteration's block, laid out slot by slot ---------------------------
  // A slot holds one MFMA plus the loads and VALU work that overlap it; a
  // scheduling fence after each slot keeps that order (the compiler would
  // otherwise cluster all exponentials ahead of the first MFMA).  Fragments
  // are loaded kAhead slots before the MFMA that uses them.
  constexpr int N_QK = NKB * NDS;           // score MFMAs of tile j+1
  constexpr int N_PV = NDB * NKB * 2;       // O MFMAs of tile j
  constexpr int NE = NKB * 16;              // probabilities per lane and tile
  constexpr int EQ = (NE + N_QK - 1) / N_QK;   // ... converted per score MFMA
  constexpr int EM = (NE + N_PV - 1) / N_PV;   // maxima taken per O MFMA
  constexpr int kAhead = 2;
  static_assert(EQ % 2 == 0 && 8 % EQ == 0 || EQ % 8 == 0, "conversion chunks must align with packs");
  bf16x8 pf[NKB][2];
  auto fused = [&](int j, f32x16 (&Scur)[NKB], f32x16 (&Snext)[NKB]) {
    const uint32_t kt_base = (uint32_t)((j + 1) % NBUF) * KT;
    const uint32_t vt_base = (uint32_t)(NBUF * KT) + (uint32_t)(j % NBUF) * VT;
    // slot i of the score MFMAs: (kb, s) = (i % NKB, i / NKB), alternating
    // accumulators; slot i of the O MFMAs: (db, kb, t) with db fastest.
    auto kslot = [&](int i) { return kfrag(kt_base, i % NKB, i / NKB); };
    auto vslot = [&](int i) {
      return vfrag(vt_base, i % NDB, (i / NDB) % NKB, i / (NDB * NKB));
    };
    bf16x8 fr[kAhead + 1];
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
    float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
    for (int i = 0; i < kAhead; ++i) fr[i] = kslot(i);
#pragma unroll
    for (int i = 0; i < N_QK; ++i) {
      const int kb = i % NKB, s = i / NKB;
      Snext[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[i % (kAhead + 1)], qf[s],
                                                          s == 0 ? f32x16{} : Snext[kb], 0, 0, 0);
      const int n = i + kAhead;
      if (n < N_QK) fr[n % (kAhead + 1)] = kslot(n);
      else fr[n % (kAhead + 1)] = vslot(n - N_QK);
#pragma unroll
      for (int e = i * EQ; e < (i + 1) * EQ && e < NE; ++e) {
        const float pvl = __builtin_amdgcn_exp2f(fmaf(Scur[e >> 4][e & 15], a.c, -m_use));
        Scur[e >> 4][e & 15] = pvl;
        if (e & 1) rs1 += pvl; else rs0 += pvl;
        if ((e & 7) == 7) {
          const int kb2 = e >> 4, t = (e >> 3) & 1;
          uint4 w;
          w.x = pack_bf16x2(Scur[kb2][8 * t + 0], Scur[kb2][8 * t + 1]);
          w.y = pack_bf16x2(Scur[kb2][8 * t + 2], Scur[kb2][8 * t + 3]);
          w.z = pack_bf16x2(Scur[kb2][8 * t + 4], Scur[kb2][8 * t + 5]);
          w.w = pack_bf16x2(Scur[kb2][8 * t + 6], Scur[kb2][8 * t + 7]);
          pf[kb2][t] = as_bf16x8(w);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    l_run += rs0 + rs1;
    float mx0 = -INFINITY, mx1 = -INFINITY;
#pragma unroll
    for (int i = 0; i < N_PV; ++i) {
      const int db = i % NDB, kb = (i / NDB) % NKB, t = i / (NDB * NKB);
      const int cur = (i + N_QK) % (kAhead + 1);
      oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[cur], pf[kb][t], oacc[db], 0, 0, 0);
      const int n = i + kAhead;
      if (n < N_PV) fr[(n + N_QK) % (kAhead + 1)] = vslot(n);
      const int e0 = i * EM;
      if (e0 < NE) rowmax_part(Snext, e0, min(EM, NE - e0), mx0, mx1);
      __builtin_amdgcn_sched_barrier(0);
    }
    // speculative maximum of tile j+1, redone after masking on boundary tiles
    cand = half_max(fmaxf(mx0, mx1)) * a.c;
  };

  // ---- prologue: tiles 0 .. NBUF-2 in flight, wait for tiles 0 and 1 --------
  if (n_steps > 0) dma(0);
  if (n_steps > 1) dma(1);
  if (NBUF == 4 && n_steps > 2) {
    dma(2);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(PER_WAVE));
  } else {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  }
  __syncthreads();
  if (n_w > 0) {
    qk(0, S0);
    rowmax(S0);
  }

  // Iteration j (j < n_w) finds S_j in Scur with its speculative maximum in
  // cand.  On its last tile a wave still computes scores of tile j+1 (from
  // whatever that buffer holds): they are never used, and the block stays
  // branch-free.
  auto iteration = [&](int j, f32x16 (&Scur)[NKB], f32x16 (&Snext)[NKB]) {
    const bool issue = j + NBUF - 1 < n_steps;
    if (issue) dma(j + NBUF - 1);
    if (j < n_w) {
      if (j >= n_full) {
        mask(Scur, j);
        rowmax(Scur);
      }
      rescale();
      fused(j, Scur, Snext);
    }
    // publish tile j+2 (read as K by iteration j+1); a DMA issued above may run on
    if (NBUF == 4 && issue) __builtin_amdgcn_s_waitcnt(vmcnt_imm(PER_WAVE));
    else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();
  };
  for (int j = 0; j < n_steps; j += 2) {
    iteration(j, S0, S1);
    if (j + 1 < n_steps) iteration(j + 1, S1, S0);
  }

  const float lt = half_sum(l_run);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  const int qrow = qw0 + l32;
  if (qrow < lq) {
    float* op = obase + (int64_t)qrow * a.o_ss + hh * 4;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float4 w;
        w.x = oacc[db][4 * g + 0] * inv;
        w.y = oacc[db][4 * g + 1] * inv;
        w.z = oacc[db][4 * g + 2] * inv;
        w.w = oacc[db][4 * g + 3] * inv;
        *reinterpret_cast<float4*>(op + db * 32 + 8 * g) = w;
      }
    if (a.lse != nullptr && hh == 0)
      a.lse[lseoff + (int64_t)h * a.lse_hs + qrow] =
          lt > 0.f ? (m_run + __log2f(lt)) * kLn2 : -INFINITY;
  }
}

// Compiled tile policies (id: waves x 32-query columns per wave, min waves
// per SIMD).  Keys per tile: 64 (32 at head_dim 256, whose output
// accumulator alone takes 128 registers per lane).
//   0: 4 waves x 1 column  (BM 128), 2 waves/SIMD -> two workgroups per CU
//   1: 2 waves x 1 column  (BM  64), for short sequences
//   2: 4 waves x 2 columns (BM 256), 1 wave/SIMD: each K/V fragment read from
//      LDS feeds two MFMAs
//   3: 8 waves x 1 column  (BM 256), 2 waves/SIMD in one workgroup
//   4: as 3, with raised wave priority while a wave issues its MFMA blocks
//   5: as 3, with 2x longer key tiles (one barrier per two sub-blocks)
//   6: as 5, with raised priority around MFMA blocks
//   7: as 0, with raised priority around MFMA blocks
//   8: ping-pong kernel, 8 waves in two alternating groups (BM 256)
//   9: 8 waves = 4 query waves x 2 key groups (BM 128): half-length key loop
//  10: 8 waves = 2 query waves x 4 key groups (BM 64, 32-key tiles)
//  11: DMA-staged kernel, 8 waves (BM 256), three buffers
//  12: DMA-staged kernel, 8 waves = 4 query waves x 2 key groups (BM 128), two buffers
//  13: DMA-staged kernel, 4 waves (BM 128), two buffers
//  14: software-pipelined kernel, 8 waves (BM 256), four buffers
//  15: software-pipelined kernel, 4 waves (BM 128), 32-key tiles, three buffers
//  16: as 15 with four buffers
//  17: DMA-staged kernel, 8 waves (BM 256), 128-key DMA tiles computed as two
//      64-key sub-tiles (one barrier per 128 keys), two buffers
//  18: DMA-staged kernel, 8 waves = 2 query waves x 4 key groups (BM 64),
//      32-key tiles, two buffers; the groups merge in two rounds
//  19: DMA-staged kernel, 8 waves (BM 256), 128-key tiles (one softmax pass
//      and one barrier per 128 keys), two buffers
//  20: as 19 with 4 waves (BM 128), two workgroups per CU
constexpr int kNumPolicies = 21;

template <int D>
constexpr int bn_for() { return D == 256 ? 32 : 64; }
template <int D>
constexpr int minw_for() { return D == 256 ? 1 : 2; }

template <int D, bool VARLEN>
hipError_t launch_d(const AttnArgs& a, int policy_id, hipStream_t stream) {
  const int64_t rows = (int64_t)a.nseq * a.hq;
  // unit-major order deals (sequence, head) units to the 8 XCDs: whole rounds of 8
  const int64_t grid = a.xcd_remap == 4
                           ? (int64_t)a.hq * a.n_vblk
                           : (a.xcd_remap == 3 ? (rows + 7) / 8 * 8 : rows) * a.n_qb * a.n_split;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  const dim3 g((unsigned)grid);
  switch (policy_id) {
    case 0:
      hipLaunchKernelGGL((attn_fwd_kernel<D, bn_for<D>(), 4, 1, minw_for<D>(), VARLEN>), g,
                         dim3(256), 0, stream, a);
      break;
    case 1:
      hipLaunchKernelGGL((attn_fwd_kernel<D, bn_for<D>(), 2, 1, minw_for<D>(), VARLEN>), g,
                         dim3(128), 0, stream, a);
      break;
    case 2:
      if constexpr (D == 256) {
        return hipErrorInvalidValue;
      } else {
        hipLaunchKernelGGL((attn_fwd_kernel<D, bn_for<D>(), 4, 2, 1, VARLEN>), g, dim3(256), 0,
                           stream, a);
      }
      break;
    case 3:
      hipLaunchKernelGGL((attn_fwd_kernel<D, bn_for<D>(), 8, 1, minw_for<D>(), VARLEN>), g,
                         dim3(512), 0, stream, a);
      break;
    case 4:
      hipLaunchKernelGGL((attn_fwd_kernel<D, bn_for<D>(), 8, 1, minw_for<D>(), VARLEN, kPrio>), g,
                         dim3(512), 0, stream, a);
      break;
    case 5:
      hipLaunchKernelGGL((attn_fwd_kernel<D, 2 * bn_for<D>(), 8, 1, minw_for<D>(), VARLEN>), g,
                         dim3(512), 0, stream, a);
      break;
    case 6:
      hipLaunchKernelGGL((attn_fwd_kernel<D, 2 * bn_for<D>(), 8, 1, minw_for<D>(), VARLEN, kPrio>),
                         g, dim3(512), 0, stream, a);
      break;
    case 7:
      hipLaunchKernelGGL((attn_fwd_kernel<D, bn_for<D>(), 4, 1, minw_for<D>(), VARLEN, kPrio>), g,
                         dim3(256), 0, stream, a);
      break;
    case 8:
      if constexpr (D == 256) {
        return hipErrorInvalidValue;
      } else {
        hipLaunchKernelGGL((attn_fwd_pingpong_kernel<D, VARLEN>), g, dim3(512), 0, stream, a);
      }
      break;
    case 9:
      if constexpr (D == 256) {
        return hipErrorInvalidValue;
      } else {
        hipLaunchKernelGGL((attn_fwd_kernel<D, 64, 8, 1, 2, VARLEN, 0, 2>), g, dim3(512), 0, stream, a);
      }
      break;
    case 10:
      if constexpr (D == 256) {
        return hipErrorInvalidValue;
      } else {
        hipLaunchKernelGGL((attn_fwd_kernel<D, 32, 8, 1, 2, VARLEN, 0, 4>), g, dim3(512), 0, stream, a);
      }
      break;
    case 11:
      if constexpr (D == 32 || D == 256) {
        return hipErrorInvalidValue;
      } else {
        hipLaunchKernelGGL((attn_fwd_dma_kernel<D, 8, 1, 3, VARLEN>), g, dim3(512), 0, stream, a);
      }
      break;
    case 12:
      if constexpr (D == 256) {
        return hipErrorInvalidValue;
      } else {
        hipLaunchKernelGGL((attn_fwd_dma_kernel<D, 8, 2, 2, VARLEN>), g, dim3(512), 0, stream, a);
      }
      break;
    case 13:
      hipLaunchKernelGGL((attn_fwd_dma_kernel<D, 4, 1, 2, VARLEN>), g, dim3(256), 0, stream, a);
      break;
    case 14:
    case 15:
    case 16:
      if constexpr (D == 256 || D == 32) {
        return hipErrorInvalidValue;
      } else {
        if (policy_id == 14)
          hipLaunchKernelGGL((attn_fwd_pipe_kernel<D, 64, 8, 4, 2, VARLEN>), g, dim3(512), 0,
                             stream, a);
        else if (policy_id == 15)
          hipLaunchKernelGGL((attn_fwd_pipe_kernel<D, 32, 4, 3, 2, VARLEN>), g, dim3(256), 0,
                             stream, a);
        else
          hipLaunchKernelGGL((attn_fwd_pipe_kernel<D, 32, 4, 4, 2, VARLEN>), g, dim3(256), 0,
                             stream, a);
      }
      break;
    case 18:
      if constexpr (D == 32 || D == 256) {
        return hipErrorInvalidValue;
      } else {
        hipLaunchKernelGGL((attn_fwd_dma_kernel<D, 8, 4, 2, VARLEN>), g, dim3(512), 0, stream, a);
      }
      break;
    case 19:
      if constexpr (D == 256) {
        return hipErrorInvalidValue;
      } else {
        hipLaunchKernelGGL((attn_fwd_dma_kernel<D, 8, 1, 2, VARLEN, 1, 1>), g, dim3(512), 0, stream, a);
      }
      break;
    case 20:
      if constexpr (D == 256) {
        return hipErrorInvalidValue;
      } else {
        hipLaunchKernelGGL((attn_fwd_dma_kernel<D, 4, 1, 2, VARLEN, 1, 1>), g, dim3(256), 0, stream, a);
      }
      break;
    case 17:
      if constexpr (D == 256) {
        return hipErrorInvalidValue;
      } else {
        hipLaunchKernelGGL((attn_fwd_dma_kernel<D, 8, 1, 2, VARLEN, 2>), g, dim3(512), 0, stream, a);
      }
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_v(const AttnArgs& a, bool varlen, int policy_id, hipStream_t stream) {
  return varlen ? launch_d<D, true>(a, policy_id, stream) : launch_d<D, false>(a, policy_id, stream);
}

}  // namespace

#ifndef ATTNFWD_D256_UNIT
bool select_policy(int head_dim, int max_seqlen_q, bool causal, int64_t rows, int override_id,
                   TilePolicy* out, int* policy_id) {
  static const TilePolicy kTable[kNumPolicies] = {{4, 1, 64}, {2, 1, 64}, {4, 2, 64}, {8, 1, 64},
                                                  {8, 1, 64}, {8, 1, 128}, {8, 1, 128}, {4, 1, 64},
                                                  {8, 1, 64}, {8, 1, 64, 2}, {8, 1, 32, 4},
                                                  {8, 1, 64}, {8, 1, 64, 2}, {4, 1, 64},
                                                  {8, 1, 64}, {4, 1, 32}, {4, 1, 32},
                                                  {8, 1, 128}, {8, 1, 32, 4}, {8, 1, 128}, {4, 1, 128}};
  int id;
  if (override_id >= 0) {
    if (override_id >= kNumPolicies) return false;
    if (head_dim == 256 && (override_id == 2 || (override_id >= 8 && override_id <= 12) ||
                            override_id >= 14))
      return false;  // not compiled (register or LDS budget)
    if (head_dim == 32 && (override_id == 11 || (override_id >= 14 && override_id <= 16) ||
                           override_id == 18))
      return false;
    if (override_id >= 19 && head_dim == 256) return false;
    id = override_id;
  } else {
    // Chosen from measured sweeps: the workload set (dense, varlen, packed,
    // grouped heads; head_dim 32..256) and grids of one sequence of 1K..8K
    // tokens with 8..64 heads, causal and not, per head_dim.  Large blocks
    // share one K/V tile among more waves but, causal, need at least two
    // rounds of workgroups over the 256 CUs: with a single round the longest
    // causal blocks run alone at the end (non-causal blocks all cost the same,
    // so one full round is enough).  With fewer blocks, key groups (18),
    // split key loops (12) or 128-key tiles at four waves (20) shorten the
    // critical path.
    const int64_t wg64 = rows * ((max_seqlen_q + 63) / 64);
    const int64_t wg128 = rows * ((max_seqlen_q + 127) / 128);
    const int64_t wg256 = rows * ((max_seqlen_q + 255) / 256);
    if (head_dim == 128 && max_seqlen_q <= 128) {
      // short packed sequences: the DMA-staged 128-query block (32 x 64:
      // 11.0 us vs 11.5 on 1; 32 slots of U{1..128}: 12.5 vs 13.8 on 0)
      id = 13;
    } else if (max_seqlen_q <= 64) {
      id = 1;  // one 64-query block covers every sequence
    } else if (max_seqlen_q < 256) {
      id = 13;
    } else if (head_dim == 128) {
      const bool few64 = max_seqlen_q >= 512 && max_seqlen_q <= 4096 &&
                         (wg64 <= 256 || (causal && wg64 <= 512 && max_seqlen_q >= 2048));
      if (wg256 >= (causal ? 512 : 256))
        id = 19;  // 128-key tiles: half the barriers and softmax passes of 11
      else if (few64)
        id = 18;  // S2048 x 16 heads causal 34 us; S4096 x 8 heads 53 vs 58 on 12
      else if (causal && max_seqlen_q <= 1024 && wg128 >= 512)
        id = 13;  // S1024 x 64 heads causal: 31 us vs 35 on 12 and 19
      else if (max_seqlen_q >= 512)
        id = 12;  // S4096 x 16 heads causal: 79 us vs 98 on 19
      else
        id = 13;
    } else if (head_dim == 64) {
      // Few 64-query blocks of 512..8192 queries: four key groups (18) or
      // two (12) shorten the longest block's loop, as at head_dim 128
      // (causal S2048 x 8 heads 18.5 us vs 27.7 on 20, S4096 x 8 heads 36.9
      // vs 50.7; non-causal S1024 x 8 heads 14.3 vs 16.1 on 20, S4096 x 8
      // heads 51.8 on 12 vs 54.4 on 20 and 57.0 on 18)
      const bool mid = max_seqlen_q >= 512 && max_seqlen_q <= 8192;
      if (mid && wg64 <= (causal ? 512 : 128))
        id = 18;
      else if (mid && !causal && wg64 <= 512)
        id = 12;
      else if (mid && causal && max_seqlen_q >= 2048 && wg64 <= 2048)
        id = 12;  // S4096 x 32 heads 90.5 us vs 97.3-104.5 on 20; S8192 x 8 heads 109.6 vs 112.5
      else if (causal)  // S1024 x 16 heads: 16 us vs 23 on 13; with more blocks 13 is up to 8 % faster
        id = wg128 <= 1024 ? 20 : 13;
      else  // S1024 x 8 heads: 15 us vs 24 on 13; ViT batch (149 x 12 heads, S1024) 593 vs 650 on 19
        id = wg256 < 256 ? 20 : wg256 < 512 ? 19 : 13;
    } else if (head_dim == 32) {
      // S1024 x 16 heads causal: 12 us vs 17 on 13; S8192 x 64 heads 402 vs 449
      id = wg256 >= (causal ? 1024 : 256) ? 19 : 20;
    } else {
      // head_dim 256 (one wave per SIMD, built with the iterative ILP
      // scheduler): the DMA-staged 128-query block beat the staged kernels
      // (0, 3) on 10 of 11 shapes from 2 x 300 to 1 x 8192 x 32 heads, causal
      // and not (1 x 4096 x 16 heads causal 186 us vs 207 on 0 and 465 on 3;
      // 4 x 2048 non-causal 348 vs 381 and 491); 8 x 1024 x 16 heads causal
      // is the exception at 172 vs 165 on 0
      id = 13;
    }
  }
  *out = kTable[id];
  if (head_dim == 256) out->bn /= 2;
  *policy_id = id;
  return true;
}

template <int D>
hipError_t merge_d(const AttnArgs& a, bool varlen, int bm, hipStream_t stream) {
  if (bm % kMergeRows != 0) return hipErrorInvalidValue;
  const int64_t grid = (int64_t)a.nseq * a.hq * a.n_qb * (bm / kMergeRows);
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  const dim3 block(kMergeRows * D / 4);
  if (varlen)
    hipLaunchKernelGGL((merge_split_kernel<D, true>), dim3((unsigned)grid), block, 0, stream, a, bm);
  else
    hipLaunchKernelGGL((merge_split_kernel<D, false>), dim3((unsigned)grid), block, 0, stream, a, bm);
  return hipGetLastError();
}

hipError_t launch_merge(const AttnArgs& a, int head_dim, bool varlen, int bm, hipStream_t stream) {
  switch (head_dim) {
    case 32: return merge_d<32>(a, varlen, bm, stream);
    case 64: return merge_d<64>(a, varlen, bm, stream);
    case 128: return merge_d<128>(a, varlen, bm, stream);
    case 256: return merge_d<256>(a, varlen, bm, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_attention(const AttnArgs& a, int head_dim, bool varlen, int policy_id,
                            hipStream_t stream) {
  switch (head_dim) {
    case 32: return launch_v<32>(a, varlen, policy_id, stream);
    case 64: return launch_v<64>(a, varlen, policy_id, stream);
    case 128: return launch_v<128>(a, varlen, policy_id, stream);
    case 256: return launch_attention_d256(a, varlen, policy_id, stream);
    default: return hipErrorInvalidValue;
  }
}

#else

// Built from attn_kernel_d256.hip: the head_dim 256 instances only.
hipError_t launch_attention_d256(const AttnArgs& a, bool varlen, int policy_id, hipStream_t stream) {
  return launch_v<256>(a, varlen, policy_id, stream);
}

#endif  // ATTNFWD_D256_UNIT

}  // namespace attnfwd
