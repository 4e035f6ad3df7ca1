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
//  * V is stored transposed in LDS (V^T[d][key]) so the A operand of the
//    second product (32 dims x 8 consecutive keys per lane) is one 16-byte
//    LDS read.  The transpose happens in registers while staging.
//  * K/V tiles are staged HBM -> registers -> LDS; the global loads of the
//    next tile are issued before the current tile's math so their latency
//    overlaps it.
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

#include <math.h>

#include <type_traits>

namespace attnfwd {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.69314718055994530942f;

__device__ __forceinline__ uint4 ld16(const uint16_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) {
  return __builtin_bit_cast(bf16x8, u);
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Buffer resource over [base, base + bytes): loads at offsets >= bytes return
// zero, which is how rows past the end of a sequence read as zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ uint4 buf_ld16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ uint32_t span_bytes(int rows, int64_t row_stride) {
  const int64_t b = (int64_t)rows * row_stride * 2;
  return b > 0xffffffffLL ? 0xffffffffu : (uint32_t)b;
}

// Key held by accumulator row i of a 32-key block (see the header comment).
__device__ __forceinline__ int key_of_row(int i) {
  return ((i >> 4) << 4) + (((i >> 2) & 1) << 3) + (((i >> 3) & 1) << 2) + (i & 3);
}

// Value of x in the other half of the wave (lane ^ 32) combined with x.
__device__ __forceinline__ float half_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 v = __builtin_convertvector(f32x2{a, b}, bf16x2);
  return __builtin_bit_cast(uint32_t, v);
}

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

template <int D, int BN, int WAVES, int QC, int MINW, bool VARLEN, int FLAGS = 0>
__global__ __launch_bounds__(WAVES * 64, MINW) void attn_fwd_kernel(const AttnArgs a) {
  constexpr int NT = WAVES * 64;
  constexpr int SUB = D == 256 ? 32 : 64;  // keys per softmax sub-block (bounds live registers)
  constexpr int NSB = BN / SUB;
  static_assert(BN % SUB == 0, "tile must hold whole sub-blocks");
  constexpr int BM = WAVES * 32 * QC;
  constexpr int PAD = 8;            // bf16 elements of padding per LDS row
  constexpr int KS = D + PAD;       // K tile row stride (keys are rows)
  constexpr int VS = BN + PAD;      // V^T tile row stride (dims are rows)
  constexpr int KT_ELEMS = BN * KS;
  constexpr int VT_ELEMS = D * VS;
  constexpr int NKB = SUB / 32;     // 32-key blocks per sub-block
  constexpr int NDS = D / 16;       // 16-dim slices of one key row
  constexpr int NDB = D / 32;       // 32-dim blocks of the output
  constexpr int K_UNITS = BN * D / 8;          // 16-byte chunks of a K tile
  constexpr int K_PER = (K_UNITS + NT - 1) / NT;
  constexpr int V_UNITS = (BN / 4) * (D / 8);  // 4 keys x 8 dims units of a V tile
  constexpr int V_PER = (V_UNITS + NT - 1) / NT;
  static_assert(BN % 32 == 0 && D % 32 == 0, "tile shape");

  // Two K/V^T buffers: tile kt+1 is written while tile kt is read.
  __shared__ __attribute__((aligned(16))) uint16_t ks[2 * KT_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t vt[2 * VT_ELEMS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
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
    const int qs = a.cu_q[seq];
    const int kst = a.cu_k[seq];
    lq = a.cu_q[seq + 1] - qs;
    lk = a.cu_k[seq + 1] - kst;
    qoff = (int64_t)qs * a.q_ss;
    koff = (int64_t)kst * a.k_ss;
    voff = (int64_t)kst * a.v_ss;
    ooff = (int64_t)qs * a.o_ss;
    lseoff = qs;
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

  const int qw0 = q0 + wave * 32 * QC;  // first query of this wave
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
      qf[c][s] = __builtin_bit_cast(bf16x8, qraw[c][s]);
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

  auto fetch = [&](int kt) {
    const uint32_t kbeg = kt * BN;
#pragma unroll
    for (int i = 0; i < K_PER; ++i) {
      const int u = tid + i * NT;
      if (K_UNITS % NT == 0 || u < K_UNITS) {
        const uint32_t row = u / (D / 8);
        const uint32_t col = (u % (D / 8)) * 8;
        kreg[i] = buf_ld16(krs, (kbeg + row) * k_row_bytes + col * 2);
      }
    }
#pragma unroll
    for (int i = 0; i < V_PER; ++i) {
      const int u = tid + i * NT;
      if (V_UNITS % NT == 0 || u < V_UNITS) {
        const uint32_t kq = u % (BN / 4);
        const uint32_t dq = u / (BN / 4);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          vreg[i][j] = buf_ld16(vrs, (kbeg + kq * 4 + j) * v_row_bytes + dq * 16);
      }
    }
  };

  auto stage = [&](int buf) {
    uint16_t* kd = ks + buf * KT_ELEMS;
    uint16_t* vd = vt + buf * VT_ELEMS;
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
        const int kq = u % (BN / 4);
        const int dq = u / (BN / 4);
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

  if (n_kt > 0) {
    fetch(0);
    stage(0);
  }
  __syncthreads();

  for (int kt = 0; kt < n_kt; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < n_kt) fetch(kt + 1);

#pragma unroll
    for (int sb = 0; sb < NSB; ++sb) {
    const int kbeg = kt * BN + sb * SUB;
    if (kbeg < kend_w) {
      const uint16_t* kd = ks + buf * KT_ELEMS + sb * SUB * KS;
      const uint16_t* vd = vt + buf * VT_ELEMS + sb * SUB;
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
#pragma unroll
        for (int c = 0; c < QC; ++c) {
          const int qi = qw0 + c * 32 + l32;
          const int lim = a.causal ? min(lk - 1, qi + off) : lk - 1;  // last visible key
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = kbeg + kb * 32 + ((r >> 3) << 4) + hh * 8 + (r & 7);
              if (key > lim) sacc[c][kb][r] = -INFINITY;
            }
          }
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
    if (kt + 1 < n_kt) stage(buf ^ 1);
    __syncthreads();
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
  const int wave = tid >> 6;
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
    const int qs = a.cu_q[seq];
    const int kst = a.cu_k[seq];
    lq = a.cu_q[seq + 1] - qs;
    lk = a.cu_k[seq + 1] - kst;
    qoff = (int64_t)qs * a.q_ss;
    koff = (int64_t)kst * a.k_ss;
    voff = (int64_t)kst * a.v_ss;
    ooff = (int64_t)qs * a.o_ss;
    lseoff = qs;
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
    qf[s] = __builtin_bit_cast(bf16x8, qraw[s]);
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
            const int lim = a.causal ? min(lk - 1, qw0 + l32 + off) : lk - 1;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int key = kbeg + kb * 32 + ((r >> 3) << 4) + hh * 8 + (r & 7);
                if (key > lim) sacc[kb][r] = -INFINITY;
              }
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
constexpr int kNumPolicies = 9;

template <int D>
constexpr int bn_for() { return D == 256 ? 32 : 64; }
template <int D>
constexpr int minw_for() { return D == 256 ? 1 : 2; }

template <int D, bool VARLEN>
hipError_t launch_d(const AttnArgs& a, int policy_id, hipStream_t stream) {
  const int64_t rows = (int64_t)a.nseq * a.hq;
  const int64_t grid = rows * a.n_qb;
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

bool select_policy(int head_dim, int max_seqlen_q, bool causal, int64_t rows, int override_id,
                   TilePolicy* out, int* policy_id) {
  static const TilePolicy kTable[kNumPolicies] = {{4, 1, 64}, {2, 1, 64}, {4, 2, 64}, {8, 1, 64},
                                                  {8, 1, 64}, {8, 1, 128}, {8, 1, 128}, {4, 1, 64},
                                                  {8, 1, 64}};
  int id;
  if (override_id >= 0) {
    if (override_id >= kNumPolicies) return false;
    if (head_dim == 256 && (override_id == 2 || override_id == 8)) return false;  // not compiled
    id = override_id;
  } else {
    // 256-query blocks share one K/V staging among eight waves, but need at
    // least one workgroup per CU (256) to fill the chip.
    const int64_t wg256 = rows * ((max_seqlen_q + 255) / 256);
    if (max_seqlen_q <= 64) {
      id = 1;  // one 64-query block covers every sequence
    } else if (head_dim == 128 && max_seqlen_q >= 256 && wg256 >= 256) {
      id = 3;
    } else if (head_dim == 64 && !causal && max_seqlen_q >= 256 && wg256 >= 256) {
      id = 3;
    } else {
      id = 0;
    }
  }
  *out = kTable[id];
  if (head_dim == 256) out->bn /= 2;
  *policy_id = id;
  return true;
}

hipError_t launch_attention(const AttnArgs& a, int head_dim, bool varlen, int policy_id,
                            hipStream_t stream) {
  switch (head_dim) {
    case 32: return launch_v<32>(a, varlen, policy_id, stream);
    case 64: return launch_v<64>(a, varlen, policy_id, stream);
    case 128: return launch_v<128>(a, varlen, policy_id, stream);
    case 256: return launch_v<256>(a, varlen, policy_id, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace attnfwd
