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
// sums use the fp32 probabilities with the same factor.  Each tile rounds P
// relative to the whole binades its maximum lies above the row's reference
// maximum (so 2^7 p < 2^8 < 448) and the PV product multiplies them back
// through its E8M0 operand scale, so the reference and O move only on a row's
// first tile or a climb of more than 32 binades.  The factors fold into the
// score scale and the final normalisation.
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

// The same product with B multiplied by 2^(scale_b - 127): each lane's E8M0
// scale applies to its own 32-element block of B, i.e. to one column.
__device__ __forceinline__ f32x16 mfma_f8_bscale(i32x8 a, i32x8 b, f32x16 c, int scale_b) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, kScaleOne, 0, scale_b);
}

// Binades a row maximum may climb above the reference m before O is rescaled
// (the PV product carries the lift meanwhile; 2^32 keeps O and l far inside
// fp32).
constexpr float kMaxLift = 32.f;

template <int D, int TK>
struct F8Tile {
  static constexpr int CPR = D / 16;    // 16-byte chunks per row
  static constexpr int R = 1024 / D;    // rows per DMA instruction
  static constexpr int NI = TK / R;     // DMA instructions per TK-row tile
  static constexpr int BYTES = TK * D;
  static __device__ __forceinline__ int swz_k(int r) {
    return D == 256 ? (r & 15)
                    : (D == 128 ? ((r >> 1) & 7) : (D == 64 ? ((r >> 2) & 3) : ((r ^ (r >> 3)) & 1)));
  }
  static __device__ __forceinline__ int swz_v(int r) {
    return D == 256 ? ((r & 7) << 1)
                    : (D == 128 ? (r & 7) : (D == 64 ? (((r >> 2) & 1) << 1) : ((r ^ (r >> 1)) & 1)));
  }
};

__device__ __forceinline__ int tile_key_of_row(int r) { return (r & ~31) + key_of_row(r & 31); }

// E4M3 bytes of four floats (round to nearest even).
__device__ __forceinline__ int pack_fp8x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

// WAVES x 32 queries per workgroup, TK keys per tile (64 or 128: one barrier,
// one row-maximum pass and one DMA wait per tile).
// Two waves per SIMD at every head_dim.  At 256 (4 waves, 64-key tiles) that
// holds with the MFMA accumulators in VGPRs (VGPR-form MFMAs, 246 registers):
// with them in AGPRs the kernel took 404 registers and copied every score
// back for the softmax.
template <int D, bool VARLEN, int WAVES, int TK>
__global__ __launch_bounds__(WAVES * 64, 2) void attn_fwd_fp8_kernel(const AttnArgs a, float o_mul) {
  using T = F8Tile<D, TK>;
  constexpr int BM = WAVES * 32;
  // fp8 MFMAs per 32x32 score block (64 dims each).  At head_dim 32 the one
  // product takes dims 0..31 from lane half 0 and zeros from lane half 1 (its
  // Q operand is 0, and its K operand repeats half 0's bytes).
  constexpr int NS = (D + 63) / 64;
  constexpr int NDB = D / 32;  // 32-dim output blocks
  constexpr int NKB = TK / 32; // 32-key score blocks per tile
  constexpr int NH = TK / 64;  // 64-key halves (one P operand each)
  __shared__ __attribute__((aligned(16))) unsigned char lds[2][2][T::BYTES];  // [buf][K|V]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  const int rows = a.nseq * a.hq;
  const int qb_rev = blockIdx.x / rows;
  int p = blockIdx.x - qb_rev * rows;
  // (sequence, head) rows spread so each XCD (workgroups are dealt round-robin
  // over 8) takes a contiguous range of heads: grouped heads share one L2
  if (a.xcd_remap) p = (p & 7) * (rows >> 3) + (p >> 3);
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
  const int q0 = qb * BM;
  if (q0 >= lq) return;
  const int kvh = h / a.group;
  const int off = lk - lq;
  int kend = lk;
  if (a.causal) kend = min(lk, q0 + BM + off);
  const int n_kt = kend > 0 ? (kend + TK - 1) / TK : 0;
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
    const uint32_t ob = (uint32_t)qrow * (uint32_t)a.q_ss + (D == 32 ? 0 : 32 * hh);
    // head_dim 32: lane half 1 carries dims 32..63, which do not exist
    const uint32_t zero_half = (D == 32 && hh == 1) ? ~0u : 0u;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(qrs, (int)(ob + 64 * s), 0, 0);
      u32x4 y = __builtin_amdgcn_raw_buffer_load_b128(qrs, (int)(ob + 64 * s + 16), 0, 0);
      asm volatile("" : "+v"(x), "+v"(y));
      x = q_sign(x, a.q_xor, a.q_clear | zero_half);
      y = q_sign(y, a.q_xor, a.q_clear | zero_half);
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
  // This wave's DMA instructions of a tile are q = wave + WAVES i; their lane
  // byte offsets inside the tile's rows are the same every tile, so they are
  // computed once, and tile t moves the buffer base by t TK rows instead
  // (scalar arithmetic): an instruction is then one M0 write and one load.
  // K rows land permuted by tile_key_of_row (the score registers then come
  // out in the order the P operand needs).
  // (head_dim 32: a tile is fewer instructions than waves; the rest issue none)
  constexpr int NP = (T::NI + WAVES - 1) / WAVES;
  static_assert(T::NI % WAVES == 0 || T::NI < WAVES, "every wave issues the same number of loads");
  uint32_t koffp[NP], voffp[NP];
  {
    const int dma_p = lane % T::CPR;
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int r = (wave + WAVES * i) * T::R + lane / T::CPR;
      koffp[i] = (uint32_t)tile_key_of_row(r) * (uint32_t)a.k_ss + 16 * (uint32_t)(dma_p ^ T::swz_k(r));
      voffp[i] = (uint32_t)r * (uint32_t)a.v_ss + 16 * (uint32_t)(dma_p ^ T::swz_v(r));
    }
  }
  // K rows of tile t into lds[t & 1][0], V rows into lds[t & 1][1]
  auto dma = [&](int t) __attribute__((always_inline)) {
    const uint32_t b = lds0 + (uint32_t)(t & 1) * 2 * T::BYTES;
    const uint32_t row0 = __builtin_amdgcn_readfirstlane(t * TK);
    const u32x4 kd = desc_advance(kdesc, row0 * (uint32_t)a.k_ss);
    const u32x4 vd = desc_advance(vdesc, row0 * (uint32_t)a.v_ss);
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int q = wave + WAVES * i;
      if (T::NI >= WAVES || q < T::NI) {
        dma16(kd, koffp[i], __builtin_amdgcn_readfirstlane(b + q * 1024));
        dma16(vd, voffp[i], __builtin_amdgcn_readfirstlane(b + T::BYTES + q * 1024));
      }
    }
  };

  // per-lane fragment offsets of the first 32-key block; block kb adds
  // 32 kb rows (the chunk swizzle depends on the row modulo 16 only)
  int k_off[2 * NS];  // [2 s + half]
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int r = l32;
      const int c = D == 32 ? half : 4 * s + 2 * hh + half;
      k_off[2 * s + half] = r * D + 16 * (c ^ T::swz_k(r));
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

  // S^T of 32-key block kb of tile t (K in lds[t & 1][0])
  auto score_block = [&](int t, int kb, f32x16& sb) __attribute__((always_inline)) {
    const unsigned char* kt = &lds[t & 1][0][0] + kb * 32 * D;
    sb = f32x16{};
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const uint4 x = *reinterpret_cast<const uint4*>(kt + k_off[2 * s]);
      const uint4 y = *reinterpret_cast<const uint4*>(kt + k_off[2 * s + 1]);
      const i32x8 af = {(int)x.x, (int)x.y, (int)x.z, (int)x.w, (int)y.x, (int)y.y, (int)y.z, (int)y.w};
      sb = mfma_f8(af, qf[s], sb);
    }
  };
  // Masks, row maximum, and the E4M3 P operands of NB 32-key score blocks
  // starting at key kbeg (register r of block b holds key
  // kbeg + 32 b + 16 (r / 8) + 8 hh + r % 8).  O and l stay relative to the
  // reference m.  P is rounded relative to mu = m + lift, lift = the whole
  // binades the tile's maximum lies above m: 2^7 p = exp2(c s - mu + 7) < 2^8
  // stays inside E4M3 (448) and is rounded four values at a time into
  // pf[b / 2] (byte 16 (b % 2) + r of a P operand <-> key
  // 32 (b % 2) + 16 (r / 8) + 8 hh + r % 8 of its 64 keys).  The PV product
  // multiplies P back by 2^lift through its E8M0 operand scale (exact), and
  // the row sum takes the same factor on the unrounded values.  m itself
  // moves (O rescaled) only on a row's first visible tile or after a climb of
  // more than kMaxLift binades.
  int psc = kScaleOne;  // E8M0 scale of this tile's P operands (127 + lift)
  auto softmax = [&](int kbeg, auto& sb, auto& pf) __attribute__((always_inline)) {
    constexpr int NB = sizeof(sb) / sizeof(sb[0]);
    const bool edge = (kbeg + 32 * NB > lk) || (a.causal && kbeg + 32 * NB - 1 > qw0 + off);
    if (edge) {
      keep_branch();
#pragma unroll
      for (int b = 0; b < NB; ++b) mask_block(sb[b], lim - kbeg - 32 * b - 8 * hh);
    }
    float mt0 = -INFINITY, mt1 = -INFINITY;  // raw score maximum (c > 0: a negative scale negates Q)
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        mt0 = fmaxf(mt0, sb[b][r]);
        mt1 = fmaxf(mt1, sb[b][r + 1]);
      }
    float mt = half_max(fmaxf(mt0, mt1)) * a.c;
    if (mt > m + kMaxLift) {
      const float alpha = __builtin_amdgcn_exp2f(m - mt);  // 0 while m = -inf
      l *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
      m = mt;
    }
    const float lift = m == -INFINITY ? 0.f : fminf(floorf(fmaxf(mt - m, 0.f)), kMaxLift);
    const float nb = m == -INFINITY ? 0.f : 7.f - (m + lift);
    psc = kScaleOne + (int)lift;
    float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int r0 = 0; r0 < 16; r0 += 4) {
        float p4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) p4[e] = __builtin_amdgcn_exp2f(fmaf(sb[b][r0 + e], a.c, nb));
        rs0 += p4[0] + p4[2];
        rs1 += p4[1] + p4[3];
        pf[b >> 1][4 * (b & 1) + (r0 >> 2)] = pack_fp8x4(p4[0], p4[1], p4[2], p4[3]);
      }
    l += ldexpf(rs0 + rs1, (int)lift);
  };
  // O^T += V^T P^T for the 64-key half hf of tile t (V in lds[t & 1][1])
  auto pv = [&](int t, int hf, const i32x8& pf) __attribute__((always_inline)) {
    const unsigned char* vt = &lds[t & 1][1][0] + hf * 64 * D;
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
      oacc[db] = mfma_f8_bscale(vf, pf, oacc[db], psc);
    }
  };

  // one barrier per tile; K and V of tile t + 1 load while tile t is processed
  if (n_kt > 0) dma(0);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __syncthreads();
  for (int t = 0; t < n_kt; ++t) {
    if (t + 1 < n_kt) dma(t + 1);
    if (t * TK < kend_w) {
      f32x16 st[NKB];
      i32x8 pf[NH];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) score_block(t, kb, st[kb]);
      softmax(t * TK, st, pf);
#pragma unroll
      for (int hf = 0; hf < NH; ++hf) pv(t, hf, pf[hf]);
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

hipError_t launch_attention_fp8(const AttnArgs& a, int head_dim, bool varlen, float o_mul, int bm,
                                hipStream_t stream) {
  const int64_t grid = (int64_t)a.nseq * a.hq * a.n_qb;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (grid == 0) return hipSuccess;
  const bool wide = bm == 256;  // a.n_qb counts blocks of bm queries
  const dim3 g((unsigned)grid), b(wide ? 512 : 256);
#define ATTN_FP8_LAUNCH(D_, V_)                                                                  \
  if (wide)                                                                                     \
    hipLaunchKernelGGL((attn_fwd_fp8_kernel<D_, V_, 8, 128>), g, b, 0, stream, a, o_mul);       \
  else                                                                                          \
    hipLaunchKernelGGL((attn_fwd_fp8_kernel<D_, V_, 4, 64>), g, b, 0, stream, a, o_mul);
  switch (head_dim) {
    case 32:
      if (varlen) { ATTN_FP8_LAUNCH(32, true) } else { ATTN_FP8_LAUNCH(32, false) }
      break;
    case 64:
      if (varlen) { ATTN_FP8_LAUNCH(64, true) } else { ATTN_FP8_LAUNCH(64, false) }
      break;
    case 128:
      if (varlen) { ATTN_FP8_LAUNCH(128, true) } else { ATTN_FP8_LAUNCH(128, false) }
      break;
    case 256:  // 128-query blocks only
      if (wide) return hipErrorInvalidValue;
      if (varlen)
        hipLaunchKernelGGL((attn_fwd_fp8_kernel<256, true, 4, 64>), g, b, 0, stream, a, o_mul);
      else
        hipLaunchKernelGGL((attn_fwd_fp8_kernel<256, false, 4, 64>), g, b, 0, stream, a, o_mul);
      break;
    default:
      return hipErrorInvalidValue;
  }
#undef ATTN_FP8_LAUNCH
  return hipGetLastError();
}

}  // namespace attnfwd
