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

template <int D, int BN, int WAVES, int QC, bool VARLEN>
__global__ __launch_bounds__(WAVES * 64) void attn_fwd_kernel(const AttnArgs a) {
  constexpr int NT = WAVES * 64;
  constexpr int BM = WAVES * 32 * QC;
  constexpr int PAD = 8;            // bf16 elements of padding per LDS row
  constexpr int KS = D + PAD;       // K tile row stride (keys are rows)
  constexpr int VS = BN + PAD;      // V^T tile row stride (dims are rows)
  constexpr int NKB = BN / 32;      // 32-key blocks per tile
  constexpr int NDS = D / 16;       // 16-dim slices of one key row
  constexpr int NDB = D / 32;       // 32-dim blocks of the output
  constexpr int K_UNITS = BN * D / 8;          // 16-byte chunks of a K tile
  constexpr int K_PER = (K_UNITS + NT - 1) / NT;
  constexpr int V_UNITS = (BN / 4) * (D / 8);  // 4 keys x 8 dims units of a V tile
  constexpr int V_PER = (V_UNITS + NT - 1) / NT;
  static_assert(BN % 32 == 0 && D % 32 == 0, "tile shape");

  __shared__ __attribute__((aligned(16))) uint16_t ks[BN * KS];
  __shared__ __attribute__((aligned(16))) uint16_t vt[D * VS];

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

  // ---- Q^T fragments (B operand), kept in registers ----------------------
  bf16x8 qf[QC][NDS];
#pragma unroll
  for (int c = 0; c < QC; ++c) {
    const int qrow = qw0 + c * 32 + l32;
    const bool ok = qrow < lq;
    const uint16_t* qp = qbase + (int64_t)(ok ? qrow : 0) * a.q_ss + hh * 8;
#pragma unroll
    for (int s = 0; s < NDS; ++s) {
      uint4 u = ok ? ld16(qp + 16 * s) : make_uint4(0, 0, 0, 0);
      qf[c][s] = as_bf16x8(u);
    }
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
    const int kbeg = kt * BN;
#pragma unroll
    for (int i = 0; i < K_PER; ++i) {
      const int u = tid + i * NT;
      if (K_UNITS % NT == 0 || u < K_UNITS) {
        const int row = u / (D / 8);
        const int col = (u % (D / 8)) * 8;
        const int key = kbeg + row;
        kreg[i] = key < lk ? ld16(kbase + (int64_t)key * a.k_ss + col) : make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < V_PER; ++i) {
      const int u = tid + i * NT;
      if (V_UNITS % NT == 0 || u < V_UNITS) {
        const int kq = u % (BN / 4);
        const int dq = u / (BN / 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int key = kbeg + kq * 4 + j;
          vreg[i][j] = key < lk ? ld16(vbase + (int64_t)key * a.v_ss + dq * 8)
                                : make_uint4(0, 0, 0, 0);
        }
      }
    }
  };

  auto stage = [&]() {
#pragma unroll
    for (int i = 0; i < K_PER; ++i) {
      const int u = tid + i * NT;
      if (K_UNITS % NT == 0 || u < K_UNITS) {
        const int row = u / (D / 8);
        const int col = (u % (D / 8)) * 8;
        *reinterpret_cast<uint4*>(ks + row * KS + col) = kreg[i];
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
          // dims dq*8+e of keys kq*4 .. kq*4+3 -> 4 consecutive bf16 of V^T row
          const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
          uint2 out;
          out.x = __builtin_amdgcn_perm(w1[e >> 1], w0[e >> 1], sel);
          out.y = __builtin_amdgcn_perm(w3[e >> 1], w2[e >> 1], sel);
          *reinterpret_cast<uint2*>(vt + (dq * 8 + e) * VS + kq * 4) = out;
        }
      }
    }
  };

  if (n_kt > 0) fetch(0);

  for (int kt = 0; kt < n_kt; ++kt) {
    stage();
    __syncthreads();
    if (kt + 1 < n_kt) fetch(kt + 1);

    const int kbeg = kt * BN;
    if (qw0 < lq && kbeg < kend_w) {
      // ---- S^T = K Q^T ------------------------------------------------------
      f32x16 sacc[QC][NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int c = 0; c < QC; ++c) sacc[c][kb] = f32x16{};
        const uint16_t* kr = ks + (kb * 32 + key_of_row(l32)) * KS + hh * 8;
#pragma unroll
        for (int s = 0; s < NDS; ++s) {
          const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kr + 16 * s);
#pragma unroll
          for (int c = 0; c < QC; ++c)
            sacc[c][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[c][s], sacc[c][kb], 0, 0, 0);
        }
      }

      // ---- mask (only tiles crossing the diagonal or the sequence end) -------
      const bool need_mask = (kbeg + BN > lk) || (a.causal && kbeg + BN - 1 > qw0 + off);
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

      // ---- online softmax (base 2) -----------------------------------------
      bf16x8 pf[QC][NKB][2];
#pragma unroll
      for (int c = 0; c < QC; ++c) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[c][kb][r]);
        mx = half_max(mx);
        const float m_new = fmaxf(m_run[c], mx * a.c);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run[c] - m_use);
        m_run[c] = m_new;
        float rs = 0.f;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float pv = __builtin_amdgcn_exp2f(fmaf(sacc[c][kb][r], a.c, -m_use));
            sacc[c][kb][r] = pv;
            rs += pv;
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
        l_run[c] = l_run[c] * alpha + rs;
#pragma unroll
        for (int db = 0; db < NDB; ++db) oacc[c][db] *= alpha;
      }

      // ---- O^T += V^T P^T ---------------------------------------------------
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const uint16_t* vr = vt + (db * 32 + l32) * VS + hh * 8;
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
    }
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

// Compiled policies.  id 0: 4 waves x 32 queries (BM 128); id 1: 2 waves x 32
// queries (BM 64) for short sequences.  Keys per tile: 64 (32 at head_dim 256,
// where the output accumulator alone takes 128 registers per lane).
constexpr int kNumPolicies = 2;

template <int D>
constexpr int bn_for() { return D == 256 ? 32 : 64; }

template <int D, bool VARLEN>
hipError_t launch_d(const AttnArgs& a, int policy_id, hipStream_t stream) {
  const int64_t rows = (int64_t)a.nseq * a.hq;
  const int64_t grid = rows * a.n_qb;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  switch (policy_id) {
    case 0:
      hipLaunchKernelGGL((attn_fwd_kernel<D, bn_for<D>(), 4, 1, VARLEN>), dim3((unsigned)grid),
                         dim3(256), 0, stream, a);
      break;
    case 1:
      hipLaunchKernelGGL((attn_fwd_kernel<D, bn_for<D>(), 2, 1, VARLEN>), dim3((unsigned)grid),
                         dim3(128), 0, stream, a);
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

bool select_policy(int head_dim, int max_seqlen_q, int override_id, TilePolicy* out, int* policy_id) {
  int id;
  if (override_id >= 0) {
    if (override_id >= kNumPolicies) return false;
    id = override_id;
  } else {
    id = max_seqlen_q <= 64 ? 1 : 0;
  }
  const int bn = head_dim == 256 ? 32 : 64;
  *out = (id == 0) ? TilePolicy{4, 1, bn} : TilePolicy{2, 1, bn};
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
