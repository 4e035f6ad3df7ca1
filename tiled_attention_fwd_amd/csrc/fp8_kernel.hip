// Attention forward on fp8 (OCP E4M3) inputs for gfx950.
//
// The pages name FP8 only as FA-3's direction (page "Lesson 5: IAW model FA2
// vs FA3 measured", closing note) and narrower KV data as a way to halve the
// bytes moved (page "why FA is 2x on A100 but 1.5x on Ascend 910", section 5).
// The computation is the attention of page "Intro to FlashAttention on Ascend
// CANN" (tiles of keys, online softmax, causal skipping) on dequantised
// values: q, k, v are E4M3 bytes with one float factor each.  Both products
// run on the fp8 MFMA (v_mfma_scale_f32_32x32x64_f8f6f4, twice the bf16
// rate): S^T = K Q^T with 64 dims per instruction, and O^T += V^T P^T with the
// probabilities rounded to E4M3 after scaling by 2^7 (the scale is folded into
// the exponent; p stays in the format's normal range down to 2^-13); the row
// sums use the fp32 probabilities with the same factor, the row maximum is
// tracked lazily (the reference moves only when passed by more than a factor
// 2, so 2^7 p <= 2^8 < 448), and the factors fold into the score scale and the
// final normalisation.
//
// Workgroup: 4 waves x 32 queries (BM 128), 64-key tiles of K and V staged by
// LDS DMA into two buffers (one barrier per tile), row-major DMA lanes with a
// 16-byte chunk swizzle: K rows (permuted with key_of_row so the score
// registers come out in the order the P operand needs) are read as 32-byte
// row fragments, V rows by ds_read_b64_tr_b8 (within a 16-lane group, lane i
// receives byte i % 8 of the 8-byte chunks addressed by lanes 2 e + i / 8).
// The fp8 MFMA pairs byte j of a lane half of A with byte j of the same lane
// half of B, so any dim (or key) order shared by both operands is valid.

#include "attn_internal.h"
#include "attn_device.h"

#include <math.h>

namespace attnfwd {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

constexpr int kScaleOne = 0x7f;  // E8M0 block scale 2^0

__device__ __forceinline__ f32x16 mfma_f8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, kScaleOne, 0, kScaleOne);
}

template <int D>
struct F8Tile {
  static constexpr int CPR = D / 16;    // 16-byte chunks per row
  static constexpr int R = 1024 / D;    // rows per DMA instruction
  static constexpr int NI = 64 / R;     // DMA instructions per 64-row tile
  static constexpr int BYTES = 64 * D;
  static __device__ __forceinline__ int swz_k(int r) { return D == 128 ? ((r >> 1) & 7) : ((r >> 2) & 3); }
  static __device__ __forceinline__ int swz_v(int r) { return D == 128 ? (r & 7) : (((r >> 2) & 1) << 1); }
};

__device__ __forceinline__ int tile_key_of_row(int r) { return (r & ~31) + key_of_row(r & 31); }

// E4M3 bytes of four floats (round to nearest even).
__device__ __forceinline__ int pack_fp8x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

template <int D, bool VARLEN>
__global__ __launch_bounds__(256, 2) void attn_fwd_fp8_kernel(const AttnArgs a, float o_mul) {
  using T = F8Tile<D>;
  constexpr int NS = D / 64;   // fp8 MFMAs per 32x32 score block
  constexpr int NDB = D / 32;  // 32-dim output blocks
  __shared__ __attribute__((aligned(16))) unsigned char lds[2][2][T::BYTES];  // [buf][K|V]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  const int rows = a.nseq * a.hq;
  const int qb_rev = blockIdx.x / rows;
  const int p = blockIdx.x - qb_rev * rows;
  const int seq = p / a.hq, h = p - seq * a.hq;
  const int qb = a.causal ? (a.n_qb - 1 - qb_rev) : qb_rev;
  const uint8_t* qp = reinterpret_cast<const uint8_t*>(a.q);
  const uint8_t* kp = reinterpret_cast<const uint8_t*>(a.k);
  const uint8_t* vp = reinterpret_cast<const uint8_t*>(a.v);
  int lq, lk;
  int64_t qrow0, krow0, obase, lbase;
  if constexpr (VARLEN) {
    const SeqRows sr = seq_rows(a, seq);
    lq = sr.lq; lk = sr.lk;
    qrow0 = sr.q_row;
    krow0 = sr.k_row;
    obase = (int64_t)sr.q_row * a.o_ss;
    lbase = (int64_t)h * a.lse_hs + sr.qs;
  } else {
    lq = a.sq; lk = a.sk;
    qrow0 = (int64_t)seq * a.sq;
    krow0 = (int64_t)seq * a.sk;
    obase = (int64_t)seq * a.o_bs;
    lbase = (int64_t)seq * a.lse_bs + (int64_t)h * a.lse_hs;
  }
  const int q0 = qb * 128;
  if (q0 >= lq) return;
  const int kvh = h / a.group;
  const int off = lk - lq;
  int kend = lk;
  if (a.causal) kend = min(lk, q0 + 128 + off);
  const int n_kt = kend > 0 ? (kend + 63) / 64 : 0;
  const int qw0 = q0 + wave * 32;
  int kend_w = lk;
  if (a.causal) kend_w = min(lk, qw0 + 32 + off);
  if (qw0 >= lq) kend_w = 0;
  const int qrow = qw0 + l32;
  const int lim = qrow >= lq ? -1 : (a.causal ? min(lk - 1, qrow + off) : lk - 1);

  // Q of this lane's query as the B operand: dims 64 s + 32 hh + 0..31
  i32x8 qf[NS];
  {
    const uint8_t* qbase = qp + qrow0 * a.q_ss + (int64_t)h * a.q_hs;
    const int64_t span = (int64_t)lq * a.q_ss;
    const __amdgpu_buffer_rsrc_t qrs =
        make_rsrc(qbase, span > 0xffffffffLL ? 0xffffffffu : (uint32_t)span);
    const uint32_t ob = (uint32_t)qrow * (uint32_t)a.q_ss + 32 * hh;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(qrs, (int)(ob + 64 * s), 0, 0);
      u32x4 y = __builtin_amdgcn_raw_buffer_load_b128(qrs, (int)(ob + 64 * s + 16), 0, 0);
      asm volatile("" : "+v"(x), "+v"(y));
      qf[s] = i32x8{(int)x[0], (int)x[1], (int)x[2], (int)x[3], (int)y[0], (int)y[1], (int)y[2], (int)y[3]};
    }
  }

  const int64_t kspan = (int64_t)lk * a.k_ss;
  const uint32_t kbytes = kspan > 0xffffffffLL ? 0xffffffffu : (uint32_t)kspan;
  const u32x4 kdesc = make_desc(kp + krow0 * a.k_ss + (int64_t)kvh * a.k_hs, kbytes);
  const int64_t vspan = (int64_t)lk * a.v_ss;
  const uint32_t vbytes = vspan > 0xffffffffLL ? 0xffffffffu : (uint32_t)vspan;
  const u32x4 vdesc = make_desc(vp + krow0 * a.v_ss + (int64_t)kvh * a.v_hs, vbytes);
  const uint32_t lds0 = lds_addr(lds);
  const int dma_p = lane % T::CPR;
  auto dma = [&](int t) {
    const uint32_t b = lds0 + (uint32_t)(t & 1) * 2 * T::BYTES;
    for (int q = wave; q < T::NI; q += 4) {
      const int r = q * T::R + lane / T::CPR;
      const uint32_t ko = (uint32_t)(t * 64 + tile_key_of_row(r)) * (uint32_t)a.k_ss +
                          16 * (uint32_t)(dma_p ^ T::swz_k(r));
      dma16(kdesc, ko, __builtin_amdgcn_readfirstlane(b + q * 1024));
      const uint32_t vo = (uint32_t)(t * 64 + r) * (uint32_t)a.v_ss +
                          16 * (uint32_t)(dma_p ^ T::swz_v(r));
      dma16(vdesc, vo, __builtin_amdgcn_readfirstlane(b + T::BYTES + q * 1024));
    }
  };

  // per-lane fragment offsets
  int k_off[2][2 * NS];  // [kb][2 s + half]
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int r = 32 * kb + l32;
        const int c = 4 * s + 2 * hh + half;
        k_off[kb][2 * s + half] = r * D + 16 * (c ^ T::swz_k(r));
      }
  const int vg = (lane >> 4) & 1, vi = lane & 15;
  int v_off[NDB][4];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int r = 16 * t + 8 * hh + (vi >> 1);
      const int c = 2 * db + vg;
      v_off[db][t] = r * D + 16 * (c ^ T::swz_v(r)) + 8 * (vi & 1);
    }

  float m = -INFINITY, l = 0.f;
  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};

  if (n_kt > 0) dma(0);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __syncthreads();
  for (int t = 0; t < n_kt; ++t) {
    if (t + 1 < n_kt) dma(t + 1);
    const int kbeg = t * 64;
    if (kbeg < kend_w) {
      const unsigned char* kt = &lds[t & 1][0][0];
      const unsigned char* vt = &lds[t & 1][1][0];
      f32x16 st[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        st[kb] = f32x16{};
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const uint4 x = *reinterpret_cast<const uint4*>(kt + k_off[kb][2 * s]);
          const uint4 y = *reinterpret_cast<const uint4*>(kt + k_off[kb][2 * s + 1]);
          const i32x8 af = {(int)x.x, (int)x.y, (int)x.z, (int)x.w, (int)y.x, (int)y.y, (int)y.z, (int)y.w};
          st[kb] = mfma_f8(af, qf[s], st[kb]);
        }
      }
      // register r of block kb holds key kbeg + 32 kb + 16 (r / 8) + 8 hh + r % 8
      const bool edge = (kbeg + 64 > lk) || (a.causal && kbeg + 63 > qw0 + off);
      float mt = -INFINITY;  // raw score maximum (scale > 0)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          if (edge) {
            const int key = kbeg + 32 * kb + ((r >> 3) << 4) + 8 * hh + (r & 7);
            if (key > lim) st[kb][r] = -INFINITY;
          }
          mt = fmaxf(mt, st[kb][r]);
        }
      mt = half_max(mt) * a.c;
      // lazy rescale: the reference m moves only when the row maximum passes
      // it by more than a factor 2, so 2^7 p <= 2^8 stays inside E4M3 (448)
      if (mt > m + 1.f) {
        const float alpha = __builtin_amdgcn_exp2f(m - mt);  // 0 while m = -inf
        l *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
        m = mt;
      }
      // 2^7 p = exp2(c s - m + 7); the row sum keeps the same factor
      const float nb = m == -INFINITY ? 0.f : 7.f - m;
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pv = __builtin_amdgcn_exp2f(fmaf(st[kb][r], a.c, nb));
          rs += pv;
          st[kb][r] = pv;
        }
      l += rs;
      // P bytes: byte 16 kb + r <-> key 32 kb + 16 (r / 8) + 8 hh + r % 8
      i32x8 pf;
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const int kb = w >> 2, r0 = 4 * (w & 3);
        pf[w] = pack_fp8x4(st[kb][r0], st[kb][r0 + 1], st[kb][r0 + 2], st[kb][r0 + 3]);
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        i32x8 vf;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          const i32x2 x = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
              (__attribute__((address_space(3))) i32x2*)(vt + v_off[db][tt]));
          vf[2 * tt] = x[0];
          vf[2 * tt + 1] = x[1];
        }
        oacc[db] = mfma_f8(vf, pf, oacc[db]);
      }
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();
  }

  l = half_sum(l);  // in units of 2^-7, like O
  if (qrow < lq) {
    const float inv = l > 0.f ? o_mul / l : 0.f;
    float* op = a.o + obase + (int64_t)qrow * a.o_ss + (int64_t)h * a.o_hs + hh * 4;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<float4*>(op + db * 32 + 8 * g) =
            make_float4(oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv, oacc[db][4 * g + 2] * inv,
                        oacc[db][4 * g + 3] * inv);
    if (a.lse != nullptr && hh == 0)
      a.lse[lbase + qrow] = l > 0.f ? (m + __log2f(l) - 7.f) * kLn2 : -INFINITY;
  }
}

}  // namespace

hipError_t launch_attention_fp8(const AttnArgs& a, int head_dim, bool varlen, float o_mul,
                                hipStream_t stream) {
  const int64_t grid = (int64_t)a.nseq * a.hq * a.n_qb;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (grid == 0) return hipSuccess;
  const dim3 g((unsigned)grid), b(256);
  switch (head_dim) {
    case 64:
      if (varlen) hipLaunchKernelGGL((attn_fwd_fp8_kernel<64, true>), g, b, 0, stream, a, o_mul);
      else hipLaunchKernelGGL((attn_fwd_fp8_kernel<64, false>), g, b, 0, stream, a, o_mul);
      break;
    case 128:
      if (varlen) hipLaunchKernelGGL((attn_fwd_fp8_kernel<128, true>), g, b, 0, stream, a, o_mul);
      else hipLaunchKernelGGL((attn_fwd_fp8_kernel<128, false>), g, b, 0, stream, a, o_mul);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace attnfwd
