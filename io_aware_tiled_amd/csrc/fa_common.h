// Shared device-side helpers of libfa (gfx950 / CDNA4 only).
//
// Matrix-core lane layouts used throughout (checked on gfx950 with an
// in-bounds probe):
//   v_mfma_f32_32x32x16_bf16  C = A(32x16) * B(16x32) + C
//     A: lane l holds A[l%32][k-slot (l/32, e)], e = 0..7   (8 bf16)
//     B: lane l holds B[k-slot (l/32, e)][l%32]            (8 bf16)
//     C: lane l register r holds C[8*(r/4) + 4*(l/32) + r%4][l%32]
//   The k-slot (l/32, e) is the same for A and B, so any consistent
//   assignment of contraction indices to slots gives the same product.
//   v_mfma_f32_32x32x2_f32: A lane l holds A[l%32][slot l/32], B likewise,
//   C as above.
//   ds_read_b64_tr_b16: inside each group of 16 lanes, lane r addresses four
//   consecutive 16-bit values M[r][0..3]; lane i receives
//   M[4e + i/4][i%4] for e = 0..3.  Pointing lane r at row (base + r/4),
//   column (cbase + 4*(r%4)) of a row-major tile gives lane i the column
//   (cbase + i) of rows base..base+3: a transposed read.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma32x2f(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Transposed 4 x 16-bit read from LDS (see the layout note above).
__device__ __forceinline__ i16x4 lds_read_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}

typedef short i16x8 __attribute__((ext_vector_type(8)));

// Concatenate two transposed reads into one MFMA operand.  Built with a
// whole-vector shuffle and bit cast: assembling a __bf16 vector element by
// element is miscompiled by the ROCm 7.2 compiler (it broadcasts element 0).
__device__ __forceinline__ bf16x8 join_bf16(i16x4 lo, i16x4 hi) {
  const i16x8 r = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, r);
}

// Halves of an 8-element bf16 vector (whole-vector shuffles, see above).
__device__ __forceinline__ bf16x4 lo4(bf16x8 x) {
  const i16x8 r = __builtin_bit_cast(i16x8, x);
  return __builtin_bit_cast(bf16x4, __builtin_shufflevector(r, r, 0, 1, 2, 3));
}
__device__ __forceinline__ bf16x4 hi4(bf16x8 x) {
  const i16x8 r = __builtin_bit_cast(i16x8, x);
  return __builtin_bit_cast(bf16x4, __builtin_shufflevector(r, r, 4, 5, 6, 7));
}

// Round-to-nearest-even float32 -> bf16 of 8 values.
__device__ __forceinline__ bf16x8 to_bf16x8(f32x8 x) {
  return __builtin_convertvector(x, bf16x8);
}

__device__ __forceinline__ bf16x4 to_bf16x4(f32x4 x) {
  return __builtin_convertvector(x, bf16x4);
}

// Index of this wavefront in its workgroup, as a wave-uniform value: the
// compiler cannot infer that threadIdx.x / 64 is uniform, and per-wave
// decisions (causal skips, tile ownership) must be scalar branches.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

// Value of the other half-wave's lane (l ^ 32).
__device__ __forceinline__ float xor32(float x) {
  return __shfl_xor(x, 32, 64);
}

// max(x[l], x[l ^ 32]) in every lane, without an LDS round trip:
// v_permlane32_swap of (x, x) yields the lower half-wave's x in the first
// result and the upper half-wave's x in the second, in every lane.
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(
      __builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x), false,
      false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]),
               __builtin_bit_cast(float, (unsigned)r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(
      __builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x), false,
      false);
  return __builtin_bit_cast(float, (unsigned)r[0]) +
         __builtin_bit_cast(float, (unsigned)r[1]);
}

// MFMA accumulating into AGPRs.  Long-lived accumulators that only MFMAs
// touch until an epilogue (dK/dV in the backward, O in the 64-row-per-
// wavefront forward) live in AGPRs, while score MFMAs of the same kernel
// write VGPRs that the VALU reads; the compiler gives all MFMAs of a kernel
// one register file, so this one is written out.  Hazards: back-to-back
// accumulation into the same AGPRs needs no wait states; any other access
// to these AGPRs (zero fill, rescale, epilogue reads) is separated from the
// MFMAs by agpr_hazard_pad().
__device__ __forceinline__ void mfma_agpr(f32x16& acc, bf16x8 a, bf16x8 b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
               : "+a"(acc)
               : "v"(a), "v"(b));
}
// Wait states between an MFMA that writes AGPRs and an instruction that
// reads them, or between a VALU write of AGPRs and an MFMA reading them as
// C, with margin: three s_nop 7 give 24.
__device__ __forceinline__ void agpr_hazard_pad() {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
}

// s_waitcnt immediate: vmcnt(0) with the LDS and export counters left free.
constexpr int kWaitVm0 = 0x0F70;

// Byte offset of an LDS location (the 32-bit LDS address).
__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return (unsigned)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// One LDS DMA: each lane loads 16 bytes at voffset through the buffer
// descriptor, and lane i's bytes land at LDS address lds + 16 i (out-of-range
// lanes load zeros).  Written out rather than through the builtin so that
// the compiler, which cannot tell the stage being filled from the stages
// being read, does not wait for the transfer before every LDS read; callers
// wait for it explicitly (vmcnt) before the barrier that publishes the
// stage.  M0 carries the LDS base: it is an operand of the statement, so
// the compiler writes it (once for consecutive transfers with one base) and
// nothing is saved or restored; the s_nop is the wait state between an M0
// write and the transfer that reads it.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rs,
                                          unsigned lds, unsigned voffset) {
  asm volatile(
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds"
      :
      : "{m0}"(lds), "v"(voffset), "s"(rs)
      : "memory");
}

// Workgroup id -> (batch-head bh, query block qb) for grids of BH heads
// times n_qblk query blocks.
__device__ __forceinline__ void block_schedule(int wg, int n_qblk, int BH,
                                               bool causal, int& bh, int& qb) {
  // Workgroups are dealt to the 8 XCDs round robin (wg % 8), each with its
  // own L2.  Consecutive ids take consecutive heads, so with BH a multiple
  // of 8 every block of a head runs on one XCD and reads K and V from one
  // L2.  Otherwise each head is split into P = 8 / gcd(BH, 8) parts
  // (alternate query blocks) so that BH P is a multiple of 8 and a head
  // spans P XCDs (when n_qblk is a multiple of P).  Causal: longest query
  // blocks first.
  int P = 8 / min(BH & -BH, 8);
  if (n_qblk % P != 0) P = 1;
  const int VH = BH * P;
  const int v = wg % VH;
  const int t = (wg / VH) * P + v % P;
  bh = v / P;
  qb = causal ? n_qblk - 1 - t : t;
}

// ---------------------------------------------------------------------------
// Attention dropout.  Random bytes come from Philox4x32-10, the counter-based
// generator of Salmon, Moraes, Dror and Shaw ("Parallel random numbers: as
// easy as 1, 2, 3", SC 2011): ten rounds map a 128-bit counter and a 64-bit
// key to four 32-bit words.  Element (b, h, i, j) uses the call with counter
// (j / 4, i / 4, b H + h, offset) and key (seed low, seed high) and reads
// byte j % 4 (least significant first) of word i % 4; it is kept iff that
// byte is >= p8 (= round(256 p)), and kept weights are scaled by
// 256 / (256 - p8).  One call thus serves a 4 x 4 block of (query, key)
// pairs.  The parameters travel as struct Dropout (fa_launch.h).

// Round r of Philox4x32 on counter x with the round key (k0, k1) advanced r
// times by the Weyl increments.
__device__ __forceinline__ void philox_round(uint32_t (&x)[4], uint32_t k0,
                                             uint32_t k1, int r) {
  const uint32_t r0 = k0 + 0x9E3779B9u * (uint32_t)r;
  const uint32_t r1 = k1 + 0xBB67AE85u * (uint32_t)r;
  const uint64_t p0 = (uint64_t)0xD2511F53u * x[0];
  const uint64_t p1 = (uint64_t)0xCD9E8D57u * x[2];
  const uint32_t n0 = (uint32_t)(p1 >> 32) ^ x[1] ^ r0;
  const uint32_t n2 = (uint32_t)(p0 >> 32) ^ x[3] ^ r1;
  x[0] = n0;
  x[1] = (uint32_t)p1;
  x[2] = n2;
  x[3] = (uint32_t)p0;
}

// Quad exchange.  Each lane of a group of four lanes (lane & 3 = w) holds
// the four words x of "its" generator call; on return x[m] holds word w of
// the call of quad lane m.  The lane first rotates its words so that the
// word lane w ^ r needs sits in slot r, the quad-permute moves bring slot r
// from lane w ^ r, and a second rotation puts them in call order.
template <int CTRL>
__device__ __forceinline__ uint32_t quad_perm(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ void quad_gather(uint32_t (&x)[4]) {
  const bool b0 = threadIdx.x & 1, b1 = threadIdx.x & 2;
  uint32_t t[4], a[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) t[r] = b0 ? x[r ^ 1] : x[r];
#pragma unroll
  for (int r = 0; r < 4; ++r) a[r] = b1 ? t[r ^ 2] : t[r];
  a[1] = quad_perm<0xB1>(a[1]);   // lanes (1, 0, 3, 2)
  a[2] = quad_perm<0x4E>(a[2]);   // lanes (2, 3, 0, 1)
  a[3] = quad_perm<0x1B>(a[3]);   // lanes (3, 2, 1, 0)
#pragma unroll
  for (int r = 0; r < 4; ++r) t[r] = b0 ? a[r ^ 1] : a[r];
#pragma unroll
  for (int r = 0; r < 4; ++r) x[r] = b1 ? t[r ^ 2] : t[r];
}

// 4 x 4 byte transpose: byte a of y[b] = byte b of x[a].
__device__ __forceinline__ void byte_transpose(uint32_t (&x)[4]) {
  uint32_t y[4];
#pragma unroll
  for (int b = 0; b < 4; ++b)
    y[b] = ((x[0] >> (8 * b)) & 0xFFu) | (((x[1] >> (8 * b)) & 0xFFu) << 8) |
           (((x[2] >> (8 * b)) & 0xFFu) << 16) | (((x[3] >> (8 * b)) & 0xFFu) << 24);
#pragma unroll
  for (int b = 0; b < 4; ++b) x[b] = y[b];
}

// Keep decision of byte b of word z.
__device__ __forceinline__ bool drop_keep(uint32_t z, int b, int p8) {
  return (int)((z >> (8 * b)) & 0xFFu) >= p8;
}

}  // namespace fa
