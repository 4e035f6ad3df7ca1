// Device helpers shared by the forward and backward attention kernels
// (gfx950): vector types, buffer descriptors, LDS DMA, the transposing LDS
// read, the MFMA row order and the chunk-major LDS tile layout.  Included by
// the kernel sources only; every definition sits in an unnamed namespace.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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

// Sign of the score scale applied to a Q fragment word by word:
// (x ^ xr) & ~clr (negation: xr = the element sign bits; zero: clr = ~0).
__device__ __forceinline__ u32x4 q_sign(u32x4 x, uint32_t xr, uint32_t clr) {
  return (x ^ xr) & ~clr;
}

// Key held by accumulator row i of a 32-key block (see the header comment).
__device__ __forceinline__ int key_of_row(int i) {
  return ((i >> 4) << 4) + (((i >> 2) & 1) << 3) + (((i >> 3) & 1) << 2) + (i & 3);
}

// Called first inside a branch on a wave-uniform condition that is rarely
// true (a tile crossing the causal diagonal or the sequence end): an empty
// volatile asm cannot be speculated, so the compiler keeps the branch instead
// of turning the masked path into selects that every tile then executes.
__device__ __forceinline__ void keep_branch() { asm volatile(""); }

// Scores of one 32-key block of the transposed score tile: register r of lane
// half hh holds key kb0 + 16 (r / 8) + 8 hh + r % 8.  Keys after `lim` (the
// lane's last visible key) get -inf.  thr = lim - kb0 - 8 hh, computed once,
// so each register costs one compare and one select.
__device__ __forceinline__ void mask_block(f32x16& s, int thr) {
#pragma unroll
  for (int r = 0; r < 16; ++r)
    if (((r >> 3) << 4) + (r & 7) > thr) s[r] = -INFINITY;
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

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ uint2 ds_read_tr16(const uint16_t* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(p));
  return __builtin_bit_cast(uint2, v);
}

// One wave-wide HBM -> LDS copy of 16 bytes per lane: lane i's bytes land at
// lds_byte_base + 16 i.  Issued through asm so the compiler does not track the
// LDS write (it would otherwise stall unrelated LDS reads on it); the kernel
// itself waits for these loads (vmcnt) before the barrier that publishes them.
// The asm has no register outputs, only inputs.
__device__ __forceinline__ void dma16(u32x4 desc, uint32_t voffset, uint32_t lds_byte_base) {
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "buffer_load_dwordx4 %0, %2, 0 offen lds"
      :
      : "v"(voffset), "s"(lds_byte_base), "s"(desc)
      : "memory", "m0");
}

// Raw buffer descriptor (same fields make_rsrc sets) as four scalars for asm.
__device__ __forceinline__ u32x4 make_desc(const void* base, uint32_t bytes) {
  const uint64_t addr = reinterpret_cast<uint64_t>(base);
  u32x4 d;
  d[0] = __builtin_amdgcn_readfirstlane((uint32_t)addr);
  d[1] = __builtin_amdgcn_readfirstlane((uint32_t)(addr >> 32) & 0xffffu);
  d[2] = __builtin_amdgcn_readfirstlane(bytes);
  d[3] = 0x00020000u;
  return d;
}

// The descriptor d (from make_desc) advanced by ofs bytes: base + ofs, and the
// range shortened by ofs (to 0 past its end), so loads relative to the new
// base still read zero beyond the original end.  Scalar arithmetic only.
__device__ __forceinline__ u32x4 desc_advance(u32x4 d, uint32_t ofs) {
  const uint64_t base = (((uint64_t)(d[1] & 0xffffu)) << 32 | d[0]) + ofs;
  u32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((uint32_t)base);
  r[1] = __builtin_amdgcn_readfirstlane((uint32_t)(base >> 32) & 0xffffu);
  r[2] = __builtin_amdgcn_readfirstlane(d[2] > ofs ? d[2] - ofs : 0u);
  r[3] = d[3];
  return r;
}

// 32-bit LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) char*)p);
}

// s_waitcnt immediate that waits until at most n vector-memory ops are in flight.
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// LDS tile layout with additive fragment addresses.  One DMA instruction moves
// 64 x 16 bytes = R = 64 / (D/8) rows of a tile; inside its 1 KiB the 16-byte
// chunk c of row-in-group i sits at slot c * R + (i ^ rot(c)) (chunk-major),
// and consecutive instructions are G bytes apart (G_K for tiles read as rows,
// G_V for tiles read transposed).  Fragment addresses are then (lane base) +
// (constant), and both read patterns are free of bank conflicts (see the
// software-pipelined forward kernel for the argument).  At head_dim 32 an
// instruction moves 16 rows; there the blocks need no padding and chunk c is
// rotated by 4 c, which keeps both read patterns of the backward's tiles free
// of bank conflicts (checked by a host model of the placement and reads).
template <int D>
struct PipeLayout {
  static constexpr int CPR = D / 8;
  static constexpr int R = 64 / CPR;
  static_assert(R == 2 || R == 4 || R == 8 || R == 16, "layout defined for head_dim 256, 128, 64 and 32");
  static constexpr int GK = 1024 + (R == 2 ? 32 : (R == 4 ? 64 : (R == 8 ? 128 : 0)));
  static constexpr int GV = 1024;
  static __device__ __forceinline__ int rot(int c) {
    return R == 8 ? 4 * ((c ^ (c >> 1)) & 1) : (R == 16 ? 4 * c : 0);
  }
  // byte offset of (row, chunk) inside a tile with instruction stride G
  static __device__ __forceinline__ int at(int row, int c, int G) {
    return (row / R) * G + 16 * (c * R + ((row % R) ^ rot(c)));
  }
};

}  // namespace
}  // namespace attnfwd
