// Microbenchmarks of the gfx950 features the attention kernels rely on:
// matrix-core (MFMA) rate on constant and on random operands, VALU issue
// cost of FMA and exp2, MFMA/VALU overlap, LDS read bandwidth for 16-byte
// row reads and transposed 8-byte reads, and LDS DMA (buffer loads that
// write LDS) from L2-resident data.
//
// Not part of libfa: a separate library (libmicro.so) that bench.py --micro
// drives.  Every kernel times itself with s_memtime (shader-clock cycles)
// and s_memrealtime (the 100 MHz constant clock), so a run reports both
// cycles per instruction and the clock the chip held.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Per-wave timing record: shader cycles and 100 MHz ticks of the timed loop.
struct Stamp {
  uint64_t cycles, ticks;
};

__device__ __forceinline__ uint64_t cyc() { return __builtin_amdgcn_s_memtime(); }
__device__ __forceinline__ uint64_t rt() { return __builtin_amdgcn_s_memrealtime(); }

// Operand of lane l for the MFMA loops: constant (every element 1.0) or
// pseudo-random bf16 bits (a hash of the lane and register index, with the
// exponent kept in [2^-8, 2^8)), built as whole 32-bit words.
__device__ bf16x8 operand(int lane, int i, bool constant) {
  u32x4 v;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    uint32_t x = 0x9E3779B9u * (uint32_t)(lane * 64 + i * 8 + e + 1);
    x ^= x >> 15;
    x *= 0x85EBCA6Bu;
    x ^= x >> 13;
    // two bf16 halves: sign, exponent 119..134, 7 mantissa bits
    const uint32_t lo = (x & 0x807Fu) | ((119u + ((x >> 8) & 15u)) << 7);
    const uint32_t hi = ((x >> 16) & 0x807Fu) | ((119u + ((x >> 24) & 15u)) << 7);
    v[e] = constant ? 0x3F803F80u : (lo | (hi << 16));
  }
  return __builtin_bit_cast(bf16x8, v);
}

// NCH independent accumulation chains of v_mfma_f32_32x32x16_bf16 per wave
// (operands fixed per chain and hidden from the compiler before the loop).
template <int NCH>
__global__ __launch_bounds__(1024) void mfma_kernel(int iters, int constant,
                                                    float* sink, Stamp* st) {
  const int lane = threadIdx.x & 63;
  bf16x8 a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = operand(lane, i, constant != 0);
    b[i] = operand(lane, i + 4, constant != 0);
    asm volatile("" : "+v"(a[i]), "+v"(b[i]));
  }
  f32x16 acc[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) acc[c] = f32x16{};
  __syncthreads();
  const uint64_t c0 = cyc(), t0 = rt();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < NCH; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[c & 3], b[c & 3],
                                                       acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < NCH; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  const uint64_t c1 = cyc(), t1 = rt();
  sink[blockIdx.x * blockDim.x + threadIdx.x] = s;
  if (lane == 0) st[(blockIdx.x * blockDim.x + threadIdx.x) >> 6] = {c1 - c0, t1 - t0};
}

// VALU issue cost: 8 independent chains of one operation per lane.
// op 0: v_fma_f32, op 1: v_exp_f32, op 2: v_add_f32.
template <int OP>
__global__ __launch_bounds__(1024) void valu_kernel(int iters, float* sink,
                                                    Stamp* st) {
  const int lane = threadIdx.x & 63;
  float x[8];
  for (int c = 0; c < 8; ++c) x[c] = 0.001f * (float)(lane + c);
  const float m = 0.999f, k = 0.0001f;
  __syncthreads();
  const uint64_t c0 = cyc(), t0 = rt();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      if (OP == 0) x[c] = __builtin_fmaf(x[c], m, k);
      if (OP == 1) x[c] = __builtin_amdgcn_exp2f(x[c]) * 0.f + x[c];   // exp + (folded) use
      if (OP == 2) x[c] = x[c] + k;
    }
    asm volatile("" : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]),
                 "+v"(x[4]), "+v"(x[5]), "+v"(x[6]), "+v"(x[7]));
  }
  const uint64_t c1 = cyc(), t1 = rt();
  float s = 0.f;
  for (int c = 0; c < 8; ++c) s += x[c];
  sink[blockIdx.x * blockDim.x + threadIdx.x] = s;
  if (lane == 0) st[(blockIdx.x * blockDim.x + threadIdx.x) >> 6] = {c1 - c0, t1 - t0};
}

// Pure exp chains (v_exp_f32 only, no multiply): 8 independent chains.
__global__ __launch_bounds__(1024) void exp_kernel(int iters, float* sink,
                                                   Stamp* st) {
  const int lane = threadIdx.x & 63;
  float x[8];
  for (int c = 0; c < 8; ++c) x[c] = -0.001f * (float)(lane + c);
  __syncthreads();
  const uint64_t c0 = cyc(), t0 = rt();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < 8; ++c) x[c] = __builtin_amdgcn_exp2f(x[c]);
    asm volatile("" : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]),
                 "+v"(x[4]), "+v"(x[5]), "+v"(x[6]), "+v"(x[7]));
  }
  const uint64_t c1 = cyc(), t1 = rt();
  float s = 0.f;
  for (int c = 0; c < 8; ++c) s += x[c];
  sink[blockIdx.x * blockDim.x + threadIdx.x] = s;
  if (lane == 0) st[(blockIdx.x * blockDim.x + threadIdx.x) >> 6] = {c1 - c0, t1 - t0};
}

// MFMA and VALU in one wave, alternating in issue order: each iteration
// issues NCH independent MFMAs, each followed by 4 independent FMAs.
__global__ __launch_bounds__(1024) void mixed_kernel(int iters, int constant,
                                                     float* sink, Stamp* st) {
  constexpr int NCH = 4;
  const int lane = threadIdx.x & 63;
  bf16x8 a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = operand(lane, i, constant != 0);
    b[i] = operand(lane, i + 4, constant != 0);
    asm volatile("" : "+v"(a[i]), "+v"(b[i]));
  }
  f32x16 acc[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) acc[c] = f32x16{};
  float x[16];
#pragma unroll
  for (int c = 0; c < 16; ++c) x[c] = 0.001f * (float)(lane + c);
  __syncthreads();
  const uint64_t c0 = cyc(), t0 = rt();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[c], b[c], acc[c], 0, 0, 0);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        x[4 * c + e] = __builtin_fmaf(x[4 * c + e], 0.999f, 0.0001f);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  const uint64_t c1 = cyc(), t1 = rt();
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < NCH; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
#pragma unroll
  for (int c = 0; c < 16; ++c) s += x[c];
  sink[blockIdx.x * blockDim.x + threadIdx.x] = s;
  if (lane == 0) st[(blockIdx.x * blockDim.x + threadIdx.x) >> 6] = {c1 - c0, t1 - t0};
}

// Issue cost of other instruction kinds between MFMAs: each iteration
// issues 4 independent MFMAs, each followed by 4 instructions of one kind.
// kind 0: s_add_u32 on independent SGPRs (SALU); 1: s_nop 0;
// 2: s_waitcnt lgkmcnt(0) with nothing outstanding; 3: ds_read_b128 (the
// results are taken once per iteration, after one wait, by an empty asm
// statement, so no other instruction is added).  Kinds 4..7 put one LDS
// operand's worth of reads after each MFMA, as the attention kernels do:
// 4: one ds_read_b128; 5: two ds_read_b64_tr_b16; 6: as 4 with the
// accumulators in AGPRs; 7: no reads, accumulators in AGPRs.  At most 2
// waves per SIMD.
template <int KIND>
__global__ __launch_bounds__(512) void issue_kernel(int iters, int constant,
                                                     float* sink, Stamp* st) {
  constexpr int NCH = 4;
  __shared__ __attribute__((aligned(16))) u32x4 buf[1024];   // 16 KB
  const int lane = threadIdx.x & 63;
  for (int i = threadIdx.x; i < 1024; i += blockDim.x)
    buf[i] = u32x4{(uint32_t)i, 1u, 2u, 3u};
  bf16x8 a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = operand(lane, i, constant != 0);
    b[i] = operand(lane, i + 4, constant != 0);
    asm volatile("" : "+v"(a[i]), "+v"(b[i]));
  }
  f32x16 acc[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) acc[c] = f32x16{};
  uint32_t s0 = 1, s1 = 2, s2 = 3, s3 = 4;
  __syncthreads();
  const uint64_t c0 = cyc(), t0 = rt();
  for (int it = 0; it < iters; ++it) {
    u32x4 r[NCH][4];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      if (KIND >= 6)
        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                     : "+a"(acc[c]) : "v"(a[c]), "v"(b[c]));
      else
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[c], b[c], acc[c], 0, 0, 0);
      if (KIND == 0) {
        asm volatile("s_add_u32 %0, %0, 1" : "+s"(s0));
        asm volatile("s_add_u32 %0, %0, 1" : "+s"(s1));
        asm volatile("s_add_u32 %0, %0, 1" : "+s"(s2));
        asm volatile("s_add_u32 %0, %0, 1" : "+s"(s3));
      } else if (KIND == 1) {
        asm volatile("s_nop 0\n\ts_nop 0\n\ts_nop 0\n\ts_nop 0");
      } else if (KIND == 2) {
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_waitcnt lgkmcnt(0)\n\t"
                     "s_waitcnt lgkmcnt(0)\n\ts_waitcnt lgkmcnt(0)" ::: "memory");
      } else if (KIND == 3) {
#pragma unroll
        for (int e = 0; e < 4; ++e) r[c][e] = buf[(lane + 64 * (4 * c + e)) & 1023];
      } else if (KIND == 4 || KIND == 6) {
        r[c][0] = buf[(lane + 64 * c) & 1023];
      } else if (KIND == 5) {
        // the forward's V operand reads: 320-byte rows, rows 0..15
        const uint16_t* tile = (const uint16_t*)&buf[0];
        const int r16 = lane & 15, dsub = (lane >> 4) & 1, hh = lane >> 5;
        const int col = 32 * (c & 3) + 16 * dsub + 4 * (r16 & 3);
        const int row = 4 * hh + (r16 >> 2);
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)&tile[row * 160 + col]);
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)&tile[(row + 8) * 160 + col]);
        r[c][0] = __builtin_bit_cast(u32x4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (KIND == 3) {
#pragma unroll
      for (int c = 0; c < NCH; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e) asm volatile("" :: "v"(r[c][e]));
    }
    if (KIND == 4 || KIND == 5 || KIND == 6) {
#pragma unroll
      for (int c = 0; c < NCH; ++c) asm volatile("" :: "v"(r[c][0]));
    }
  }
  if (KIND >= 6) asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  const uint64_t c1 = cyc(), t1 = rt();
  float s = (float)(s0 + s1 + s2 + s3);
#pragma unroll
  for (int c = 0; c < NCH; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  sink[blockIdx.x * blockDim.x + threadIdx.x] = s;
  if (lane == 0) st[(blockIdx.x * blockDim.x + threadIdx.x) >> 6] = {c1 - c0, t1 - t0};
}

// v_mfma_f32_16x16x32_bf16 chains fed from LDS through a four-deep operand
// ring, as the attention kernels feed theirs (the compiler waits for each
// operand before its MFMA): KIND 0 register operands only; 1 one
// ds_read_b128 (16-byte row read, B operand layout: lane l reads row l % 16,
// elements 8 (l / 16) .. + 8 of a 32-element slice) per MFMA; 2 two
// ds_read_b64_tr_b16 (the transposed reads) per MFMA; 3 the two
// alternating, the backward's mix.  Rows of 304 bytes (the backward's
// stride), 64 rows; every read stays inside the tile.
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int KIND>
__global__ __launch_bounds__(512) void issue16_kernel(int iters, int constant,
                                                      float* sink, Stamp* st) {
  constexpr int S = 152;   // elements per row
  __shared__ __attribute__((aligned(16))) uint16_t tile[64 * S];
  // finite bf16 values in [2^-7, 2^-5)
  for (int i = threadIdx.x; i < 64 * S; i += blockDim.x)
    tile[i] = (uint16_t)(0x3C00u | (((uint32_t)i * 0x9E37u) >> 3 & 0x1FFu));
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int r16 = lane & 15, g4 = lane >> 4, hh = lane >> 5;
  const int dsub = (lane >> 4) & 1;
  bf16x8 a[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) a[c] = operand(lane, c, constant != 0);
  f32x4 acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto fetch = [&](int k, int it) -> bf16x8 {
    const bool tr = KIND == 2 || (KIND == 3 && (k & 1));
    if (!tr) {
      const int row = (((k >> 2) + it + w) & 3) * 16 + r16;     // <= 63
      const int col = 32 * (k & 3) + 8 * g4;                     // <= 120 (+8)
      return *(const bf16x8*)&tile[row * S + col];
    }
    const int col = 32 * (k & 3) + 16 * dsub + 4 * (r16 & 3);    // <= 124 (+4)
    const int row = (((k >> 2) + it) & 1) * 32 + 4 * hh + (r16 >> 2);   // <= 39 (+8)
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)&tile[row * S + col]);
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)&tile[(row + 8) * S + col]);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  bf16x8 op[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) op[k] = KIND == 0 ? a[k] : fetch(k, 0);
  __syncthreads();
  const uint64_t c0 = cyc(), t0 = rt();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int c = k & 3;
      if (KIND == 0) {
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[c], a[(c + 1) & 3], acc[c], 0, 0, 0);
      } else {
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[c], op[k & 3], acc[c], 0, 0, 0);
        op[k & 3] = fetch((k + 4) & 15, it + ((k + 4) >> 4));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  const uint64_t c1 = cyc(), t1 = rt();
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int r = 0; r < 4; ++r) s += acc[c][r];
#pragma unroll
  for (int k = 0; k < 4; ++k) s += (float)op[k][0];
  sink[blockIdx.x * blockDim.x + threadIdx.x] = s;
  if (lane == 0) st[(blockIdx.x * blockDim.x + threadIdx.x) >> 6] = {c1 - c0, t1 - t0};
}

// The same for v_mfma_f32_32x32x16_bf16 (the kernels' shape): four chains
// fed through a four-deep operand ring from 304-byte rows; KIND 1 one
// ds_read_b128 per MFMA (lane l reads row l % 32, elements 8 (l / 32) .. + 8
// of a 16-element slice), 2 two ds_read_b64_tr_b16, 3 the two alternating.
template <int KIND>
__global__ __launch_bounds__(512) void issue32r_kernel(int iters, int constant,
                                                       float* sink, Stamp* st) {
  constexpr int S = 152;
  __shared__ __attribute__((aligned(16))) uint16_t tile[64 * S];
  for (int i = threadIdx.x; i < 64 * S; i += blockDim.x)
    tile[i] = (uint16_t)(0x3C00u | (((uint32_t)i * 0x9E37u) >> 3 & 0x1FFu));
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int l32 = lane & 31, r16 = lane & 15, hh = lane >> 5;
  const int dsub = (lane >> 4) & 1;
  bf16x8 a[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) a[c] = operand(lane, c, constant != 0);
  f32x16 acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) acc[c] = f32x16{};
  auto fetch = [&](int k, int it) -> bf16x8 {
    const bool tr = KIND == 2 || (KIND == 3 && (k & 1));
    if (!tr) {
      const int row = (((k >> 3) + it + w) & 1) * 32 + l32;      // <= 63
      const int col = 16 * (k & 7) + 8 * hh;                     // <= 120 (+8)
      return *(const bf16x8*)&tile[row * S + col];
    }
    const int col = 32 * (k & 3) + 16 * dsub + 4 * (r16 & 3);    // <= 124 (+4)
    const int row = (((k >> 2) + it) & 1) * 32 + 4 * hh + (r16 >> 2);   // <= 39 (+8)
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)&tile[row * S + col]);
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)&tile[(row + 8) * S + col]);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  bf16x8 op[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) op[k] = fetch(k, 0);
  __syncthreads();
  const uint64_t c0 = cyc(), t0 = rt();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int c = k & 3;
      acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[c], op[k & 3], acc[c], 0, 0, 0);
      op[k & 3] = fetch((k + 4) & 15, it + ((k + 4) >> 4));
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  const uint64_t c1 = cyc(), t1 = rt();
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
#pragma unroll
  for (int k = 0; k < 4; ++k) s += (float)op[k][0];
  sink[blockIdx.x * blockDim.x + threadIdx.x] = s;
  if (lane == 0) st[(blockIdx.x * blockDim.x + threadIdx.x) >> 6] = {c1 - c0, t1 - t0};
}

// LDS read bandwidth.  kind 0: ds_read_b128 of 16-byte row slices (lane l
// reads row l % 32 of a 32-row tile with a 272-byte padded stride, half
// (l / 32) of a 32-byte slice: the attention kernels' K operand reads);
// kind 1: pairs of ds_read_b64_tr_b16 (the transposed V operand reads) on
// 320-byte rows, the forward's V stride.  8 operands per wave per
// iteration.  STRIDE (elements per row) defaults to the forward's strides;
// 152 (304-byte rows) is the backward's, shared by both read kinds.
constexpr int kLdsRows = 64;

template <int KIND, int STRIDE = (KIND == 0 ? 136 : 160)>
__global__ __launch_bounds__(1024) void lds_kernel(int iters, float* sink,
                                                   Stamp* st) {
  constexpr int kLdsStride = STRIDE;   // elements per row
  __shared__ __attribute__((aligned(16))) uint16_t tile[kLdsRows * kLdsStride];
  for (int i = threadIdx.x; i < kLdsRows * kLdsStride; i += blockDim.x)
    tile[i] = (uint16_t)(i * 7);
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  u32x4 acc = u32x4{0, 0, 0, 0};
  const int l32 = lane & 31, hh = lane >> 5, r16 = lane & 15;
  const int dsub = (lane >> 4) & 1;
  const uint64_t c0 = cyc(), t0 = rt();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int base = ((w + u + it) & 1) * 32;
      if (KIND == 0) {
        const uint16_t* p = &tile[(base + l32) * kLdsStride + 16 * (u & 7) + 8 * hh];
        acc ^= *(const u32x4*)p;
      } else {
        const int col = 32 * (u & 3) + 16 * dsub + 4 * (r16 & 3);
        const int row = (((u >> 2) + it) & 1) * 32 + 4 * hh + (r16 >> 2);
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)&tile[row * kLdsStride + col]);
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)&tile[(row + 8) * kLdsStride + col]);
        acc ^= __builtin_bit_cast(u32x4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    }
  }
  const uint64_t c1 = cyc(), t1 = rt();
  sink[blockIdx.x * blockDim.x + threadIdx.x] =
      (float)(acc[0] ^ acc[1] ^ acc[2] ^ acc[3]);
  if (lane == 0) st[(blockIdx.x * blockDim.x + threadIdx.x) >> 6] = {c1 - c0, t1 - t0};
}

// LDS DMA: each wave repeatedly loads 1 KB per instruction (64 lanes x 16
// bytes) from a 64 KB global buffer (L2-resident after the first pass)
// straight into LDS, NQ instructions in flight before each wait.
__global__ __launch_bounds__(1024) void dma_kernel(const uint16_t* src,
                                                   int iters, float* sink,
                                                   Stamp* st) {
  __shared__ __attribute__((aligned(16))) uint16_t buf[16][512];   // 16 KB
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const auto rs = __builtin_amdgcn_make_buffer_rsrc((void*)src, (short)0,
                                                    65536, 0x00020000);
  const unsigned lds0 =
      (unsigned)(uintptr_t)(const __attribute__((address_space(3))) void*)&buf[0][0];
  const uint64_t c0 = cyc(), t0 = rt();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const unsigned lds = lds0 + 1024u * ((w * 8 + u) & 15);
      const unsigned voff = (unsigned)((((it * 8 + u) * 64 + w * 512) % 4096) * 16 + lane * 16) % 65536u;
      unsigned saved;
      asm volatile(
          "s_mov_b32 %0, m0\n\t"
          "s_mov_b32 m0, %1\n\t"
          "s_nop 0\n\t"
          "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
          "s_mov_b32 m0, %0"
          : "=&s"(saved)
          : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(rs)
          : "memory");
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  const uint64_t c1 = cyc(), t1 = rt();
  __syncthreads();
  sink[blockIdx.x * blockDim.x + threadIdx.x] = (float)buf[lane & 15][w];
  if (lane == 0) st[(blockIdx.x * blockDim.x + threadIdx.x) >> 6] = {c1 - c0, t1 - t0};
}

}  // namespace

// Runs one microbenchmark on the current device: `which` selects the kernel
// (0 MFMA 1 chain, 1 MFMA 4 chains, 2 FMA, 3 exp2, 4 add, 5 MFMA+FMA mixed,
// 6 LDS row reads, 7 LDS transposed reads, 8 LDS DMA, 9 exp-only chains,
// 10..13 MFMA + 4 SALU / s_nop / s_waitcnt / ds_read_b128 after each,
// 14..17 MFMA + one operand of LDS reads, see issue_kernel, 18 and 19 as
// 6 and 7 on the backward's 304-byte rows, 20..23 16x16x32 MFMA chains
// fed from LDS, see issue16_kernel, 24..26 the same for 32x32x16, see
// issue32r_kernel),
// `wps` wavefronts per SIMD (one workgroup of 256 wps threads per CU over
// `cus` CUs), `constant` the MFMA operand kind.  Outputs: mean shader cycles
// and mean microseconds of the timed loop per wavefront, and the kernel time
// in ms (hipEvent).  Returns 0 or a HIP error code.
extern "C" int micro_run(int which, int wps, int constant, int iters, int cus,
                         double* cycles, double* us, double* kernel_ms) {
  const int threads = 256 * wps;
  const int waves = cus * 4 * wps;
  float* sink = nullptr;
  Stamp* st = nullptr;
  uint16_t* src = nullptr;
  hipError_t e = hipMalloc(&sink, (size_t)cus * threads * sizeof(float));
  if (e == hipSuccess) e = hipMalloc(&st, (size_t)waves * sizeof(Stamp));
  if (e == hipSuccess) e = hipMalloc(&src, 65536);
  if (e == hipSuccess) e = hipMemset(src, 0, 65536);
  hipEvent_t ev0, ev1;
  if (e == hipSuccess) e = hipEventCreate(&ev0);
  if (e == hipSuccess) e = hipEventCreate(&ev1);
  if (e != hipSuccess) return (int)e;
  auto launch = [&]() {
    const dim3 g(cus), b(threads);
    switch (which) {
      case 0: hipLaunchKernelGGL(mfma_kernel<1>, g, b, 0, 0, iters, constant, sink, st); break;
      case 1: hipLaunchKernelGGL(mfma_kernel<4>, g, b, 0, 0, iters, constant, sink, st); break;
      case 2: hipLaunchKernelGGL(valu_kernel<0>, g, b, 0, 0, iters, sink, st); break;
      case 3: hipLaunchKernelGGL(valu_kernel<1>, g, b, 0, 0, iters, sink, st); break;
      case 4: hipLaunchKernelGGL(valu_kernel<2>, g, b, 0, 0, iters, sink, st); break;
      case 5: hipLaunchKernelGGL(mixed_kernel, g, b, 0, 0, iters, constant, sink, st); break;
      case 6: hipLaunchKernelGGL(lds_kernel<0>, g, b, 0, 0, iters, sink, st); break;
      case 7: hipLaunchKernelGGL(lds_kernel<1>, g, b, 0, 0, iters, sink, st); break;
      case 8: hipLaunchKernelGGL(dma_kernel, g, b, 0, 0, src, iters, sink, st); break;
      case 9: hipLaunchKernelGGL(exp_kernel, g, b, 0, 0, iters, sink, st); break;
      case 10: hipLaunchKernelGGL(issue_kernel<0>, g, b, 0, 0, iters, constant, sink, st); break;
      case 11: hipLaunchKernelGGL(issue_kernel<1>, g, b, 0, 0, iters, constant, sink, st); break;
      case 12: hipLaunchKernelGGL(issue_kernel<2>, g, b, 0, 0, iters, constant, sink, st); break;
      case 13: hipLaunchKernelGGL(issue_kernel<3>, g, b, 0, 0, iters, constant, sink, st); break;
      case 14: hipLaunchKernelGGL(issue_kernel<4>, g, b, 0, 0, iters, constant, sink, st); break;
      case 15: hipLaunchKernelGGL(issue_kernel<5>, g, b, 0, 0, iters, constant, sink, st); break;
      case 16: hipLaunchKernelGGL(issue_kernel<6>, g, b, 0, 0, iters, constant, sink, st); break;
      case 17: hipLaunchKernelGGL(issue_kernel<7>, g, b, 0, 0, iters, constant, sink, st); break;
      case 18: hipLaunchKernelGGL((lds_kernel<0, 152>), g, b, 0, 0, iters, sink, st); break;
      case 19: hipLaunchKernelGGL((lds_kernel<1, 152>), g, b, 0, 0, iters, sink, st); break;
      case 20: hipLaunchKernelGGL(issue16_kernel<0>, g, b, 0, 0, iters, constant, sink, st); break;
      case 21: hipLaunchKernelGGL(issue16_kernel<1>, g, b, 0, 0, iters, constant, sink, st); break;
      case 22: hipLaunchKernelGGL(issue16_kernel<2>, g, b, 0, 0, iters, constant, sink, st); break;
      case 23: hipLaunchKernelGGL(issue16_kernel<3>, g, b, 0, 0, iters, constant, sink, st); break;
      case 24: hipLaunchKernelGGL(issue32r_kernel<1>, g, b, 0, 0, iters, constant, sink, st); break;
      case 25: hipLaunchKernelGGL(issue32r_kernel<2>, g, b, 0, 0, iters, constant, sink, st); break;
      case 26: hipLaunchKernelGGL(issue32r_kernel<3>, g, b, 0, 0, iters, constant, sink, st); break;
      default: break;
    }
  };
  launch();   // warm-up
  e = hipDeviceSynchronize();
  if (e == hipSuccess) {
    hipEventRecord(ev0, 0);
    launch();
    hipEventRecord(ev1, 0);
    e = hipDeviceSynchronize();
  }
  float ms = 0.f;
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, ev0, ev1);
  Stamp* h = new Stamp[waves];
  if (e == hipSuccess)
    e = hipMemcpy(h, st, (size_t)waves * sizeof(Stamp), hipMemcpyDeviceToHost);
  if (e == hipSuccess) {
    double c = 0, t = 0;
    for (int i = 0; i < waves; ++i) {
      c += (double)h[i].cycles;
      t += (double)h[i].ticks;
    }
    *cycles = c / waves;
    *us = t / waves / 100.0;   // 100 MHz ticks
    *kernel_ms = ms;
  }
  delete[] h;
  hipEventDestroy(ev0);
  hipEventDestroy(ev1);
  hipFree(sink);
  hipFree(st);
  hipFree(src);
  return (int)e;
}
