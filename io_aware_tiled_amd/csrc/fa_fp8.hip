// FP8 forward of libfa with incoherent processing, for gfx950 (CDNA4).
//
// Page cited: [MM] "Is a full-day context better than a 10-minute context?
// Flash attention and the sequence-length question" (marketmaker.cc blog),
// section "FA3: Hopper", item 3: FP8 attention is hurt by outliers; rotating
// the vectors at random before block-wise quantisation spreads an outlier
// over all coordinates and lowers the error.  The readings (randomised
// Hadamard rotation of Q and K, 32-value power-of-two block scales, E4M3
// codes) and the workspace layout are stated in include/fa.h.
//
// Two steps:
//   1. Quantisation (HBM-bound, one launch): each row of Q and K is rotated
//      with the fast Walsh-Hadamard transform (float32, one lane per 32
//      coordinates, stages in order) and written as E4M3 codes plus one
//      E8M0 scale byte per 32 coordinates; each 64-key tile of V is staged
//      through LDS and written transposed (channel-major) with a scale byte
//      per 32 keys.  K rows are
//      permuted inside each 64-key tile so that the score accumulator hands
//      every lane the keys its P operand needs (below).
//   2. Attention: the online softmax of the bf16 kernels, with both matrix
//      products on v_mfma_scale_f32_32x32x64_f8f6f4, whose per-lane E8M0
//      scales are the block scales.  On that instruction a lane supplies 32
//      bytes of the contraction, bytes 0-15 in 32-value block 0 and bytes
//      16-31 in block 1; lanes l and l + 32 supply the scales of blocks 0
//      and 1 of row l.  So a Q or K lane of half-wave u holds coordinates
//      [64m + 16u, +16) and [64m + 32 + 16u, +16) for MFMA m, and its scale
//      byte m is that of block 2m + u.  For O^T += V^T P^T the contraction is
//      the 64 keys of a tile: a lane of half-wave u holds keys [16u, +16)
//      and [32 + 16u, +16), which are exactly the keys of that lane's S^T
//      accumulator registers thanks to the K row permutation, so P^T is
//      packed to E4M3 in place (scale 1) and V^T comes from its
//      channel-major tile with two 16-byte LDS reads.
#include "fa.h"
#include "fa_common.h"
#include "fa_launch.h"


namespace fa {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kBC = 64;          // keys per tile
constexpr int kNW = 4;           // wavefronts per attention workgroup
constexpr int kBR = 32 * kNW;    // query rows per attention workgroup
constexpr int kNS = 4;           // LDS stages of the K/V ring
constexpr int kVRB = FA_FP8_V_ROW_BYTES;
// Largest lane sum of weights accepted against a stale reference; it also
// bounds every weight, so the E4M3 codes of P (largest finite 448) never
// overflow.
constexpr float kSumLimit = 0x1p8f;
constexpr unsigned kE8M0One = 127u;   // scale byte of 2^0

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float((unsigned)b << 16);
}

// E8M0 exponent of a 32-value block: the smallest e with amax <= 448 * 2^e,
// clamped to [-127, 127] (zero, subnormal amax: -127).  448 = 1.75 * 2^8,
// so e = E - 8 when amax's mantissa is at most 1.75, else E - 7.
__device__ __forceinline__ int block_exponent(float amax) {
  const unsigned u = __float_as_uint(amax);
  const int ef = (int)(u >> 23);
  if (ef == 0) return -127;
  const int E = ef - 127;
  const int e = (u & 0x7FFFFFu) <= 0x600000u ? E - 8 : E - 7;
  return max(-127, min(127, e));
}

// 2^-e as a float (e in [-127, 120] for finite inputs: a normal number).
__device__ __forceinline__ float pow2_neg(int e) {
  return __uint_as_float((unsigned)(127 - e) << 23);
}

// Four float32 -> four E4M3 bytes (round to nearest even) in one dword.
__device__ __forceinline__ unsigned pack_fp8x4(float a, float b, float c,
                                               float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (unsigned)w;
}

// ---------------------------------------------------------------------------
// Step 1: one launch quantises Q, K and V.  Workgroups [0, nrb) take rows of
// Q, [nrb, 2 nrb) rows of K, the rest 64-key tiles of V.
constexpr int kQThreads = 256;

// One row of Q or K: D/32 lanes, lane li owning coordinates [32 li, +32)
// (one scale block).  Walsh-Hadamard stages t = 0..4 inside the lane, then
// t = 5 (and 6) across lanes: the lower coordinate of a pair becomes a + b,
// the upper a - b, in float32, in stage order.
template <int D, bool PERMUTE>
__device__ __forceinline__ void quant_row(const uint16_t* __restrict__ src,
                                          const int8_t* __restrict__ signs,
                                          uint8_t* __restrict__ dst, int N,
                                          int Np, long long grow, bool live) {
  constexpr int LPR = D / 32;
  constexpr int RB = FA_FP8_ROW_BYTES(D);
  const int lane = threadIdx.x & 63;
  const int li = lane % LPR;
  const long long bh = live ? grow / Np : 0;
  const int n = live ? (int)(grow % Np) : 0;

  float x[32];
  if (live && n < N) {
    const uint16_t* srow = src + ((size_t)bh * N + n) * D + 32 * li;
    u32x4 raw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) raw[i] = *(const u32x4*)(srow + 8 * i);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        x[8 * i + 2 * c] = __uint_as_float(raw[i][c] << 16);
        x[8 * i + 2 * c + 1] = __uint_as_float(raw[i][c] & 0xFFFF0000u);
      }
  } else {
#pragma unroll
    for (int e = 0; e < 32; ++e) x[e] = 0.f;
  }

  if (signs != nullptr) {
#pragma unroll
    for (int e = 0; e < 32; ++e)
      if (signs[32 * li + e] < 0) x[e] = -x[e];
#pragma unroll
    for (int h = 1; h < 32; h *= 2) {
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        if ((e & h) == 0) {
          const float a = x[e], b = x[e + h];
          x[e] = a + b;
          x[e + h] = a - b;
        }
      }
    }
#pragma unroll
    for (int lb = 1; lb < LPR; lb *= 2) {
      const bool upper = (li & lb) != 0;
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        const float p = __shfl_xor(x[e], lb, 64);
        x[e] = upper ? p - x[e] : x[e] + p;
      }
    }
  }

  float am = 0.f;
#pragma unroll
  for (int e = 0; e < 32; ++e) am = fmaxf(am, fabsf(x[e]));
  const int ex = block_exponent(am);
  const float inv = pow2_neg(ex);
  u32x4 codes[2];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    codes[i / 4][i % 4] = pack_fp8x4(x[4 * i] * inv, x[4 * i + 1] * inv,
                                     x[4 * i + 2] * inv, x[4 * i + 3] * inv);
  // Scale bytes, gathered by the row's first lane: byte u (D/64) + m is the
  // scale of block 2m + u.
  const unsigned sbyte = (unsigned)(ex + 127);
  unsigned tail = 0;
#pragma unroll
  for (int blk = 0; blk < LPR; ++blk) {
    const unsigned sb = (unsigned)__shfl((int)sbyte, lane - li + blk, 64);
    tail |= sb << (8 * ((blk % 2) * (D / 64) + blk / 2));
  }
  if (!live) return;
  int row = n;
  if (PERMUTE) {
    // key 64j + 32t + 16u + r  ->  row 64j + 32t + 8(r/4) + 4u + r%4
    const int kt = n & 63, t = kt >> 5, u = (kt >> 4) & 1, r = kt & 15;
    row = (n & ~63) + 32 * t + 8 * (r >> 2) + 4 * u + (r & 3);
  }
  uint8_t* drow = dst + ((size_t)bh * Np + row) * RB;
  *(u32x4*)(drow + 32 * li) = codes[0];
  *(u32x4*)(drow + 32 * li + 16) = codes[1];
  if (li == 0) *(u32x4*)(drow + D) = u32x4{tail, 0u, 0u, 0u};
}

template <int D>
__global__ __launch_bounds__(kQThreads) void fp8_quant_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int8_t* __restrict__ signs,
    uint8_t* __restrict__ q8, uint8_t* __restrict__ k8,
    uint8_t* __restrict__ v8, int N, int Np, long long rows, int nrb) {
  constexpr int RPB = kQThreads / (D / 32);     // rows per workgroup
  constexpr int TPW = kQThreads / (2 * D);      // V tiles per workgroup
  constexpr int VST = D + 8;                    // LDS row stride (bf16)
  __shared__ __attribute__((aligned(16))) uint16_t tile[TPW][kBC * VST];
  const int tid = threadIdx.x;
  const int wg = blockIdx.x;
  if (wg < 2 * nrb) {
    const bool is_k = wg >= nrb;
    const long long grow = (long long)(is_k ? wg - nrb : wg) * RPB + tid / (D / 32);
    const bool live = grow < rows;
    if (is_k) quant_row<D, true>(k, signs, k8, N, Np, grow, live);
    else quant_row<D, false>(q, signs, q8, N, Np, grow, live);
    return;
  }
  // V: tile (bh, j); coalesced 16-byte loads of the 64 x D bf16 tile into
  // LDS, then thread (c, u) quantises channel c, keys 32u .. 32u + 31.
  const int ntiles = Np / kBC;
  const long long vt = (long long)(wg - 2 * nrb) * TPW + tid / (2 * D);
  const long long nvt = rows / kBC;
  const int sub = tid / (2 * D);
  const int ltid = tid % (2 * D);
  const bool live = vt < nvt;
  const long long bh = live ? vt / ntiles : 0;
  const int j = live ? (int)(vt % ntiles) : 0;
  const uint16_t* vh = v + (size_t)bh * N * D;
  constexpr int CPT = kBC * D / 8 / (2 * D);    // 16-byte chunks per thread
#pragma unroll
  for (int r = 0; r < CPT; ++r) {
    const int c = ltid + 2 * D * r;
    const int row = c / (D / 8), col = 8 * (c % (D / 8));
    const int key = j * kBC + row;
    u32x4 val = u32x4{0u, 0u, 0u, 0u};
    if (live && key < N) val = *(const u32x4*)(vh + (size_t)key * D + col);
    *(u32x4*)(&tile[sub][row * VST + col]) = val;
  }
  __syncthreads();
  if (!live) return;
  const int c = ltid >> 1, u = ltid & 1;
  float x[32];
#pragma unroll
  for (int i = 0; i < 32; ++i)
    x[i] = bf16_to_f32(tile[sub][(32 * u + i) * VST + c]);
  float am = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) am = fmaxf(am, fabsf(x[i]));
  const int ex = block_exponent(am);
  const float inv = pow2_neg(ex);
  u32x4 w[2];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    w[i / 4][i % 4] = pack_fp8x4(x[4 * i] * inv, x[4 * i + 1] * inv,
                                 x[4 * i + 2] * inv, x[4 * i + 3] * inv);
  uint8_t* drow = v8 + (((size_t)bh * ntiles + j) * D + c) * kVRB;
  *(u32x4*)(drow + 32 * u) = w[0];
  *(u32x4*)(drow + 32 * u + 16) = w[1];
  const unsigned s0 = (unsigned)(ex + 127);
  const unsigned s1 = (unsigned)__shfl_xor((int)s0, 1, 64);
  if (u == 0) *(u32x4*)(drow + 64) = u32x4{s0 | (s1 << 8), 0u, 0u, 0u};
}

// ---------------------------------------------------------------------------
// Step 2: attention on the quantised operands.  One workgroup = 4
// wavefronts = 128 query rows (32 per wavefront, one query per lane pair),
// two workgroups per CU: the two wavefronts on a SIMD belong to different
// workgroups, so their matrix-core and VALU phases drift apart and overlap
// (a software pipeline inside each wavefront, as in the bf16 kernels,
// measured slower here: it needs the score registers of two tiles).  K and
// V tiles go from HBM to LDS by DMA through four stages, tile j issuing
// tile j + 3, one barrier per tile.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t byte_rsrc(const uint8_t* p,
                                                            int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)p, (short)0, bytes,
                                           0x00020000);
}

template <int M>
__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c,
                                           unsigned sa, unsigned sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
      a, b, c, 0, 0, M, (int)sa, M, (int)sb);
}

__device__ __forceinline__ i32x8 join8(u32x4 lo, u32x4 hi) {
  const u32x4 l = lo, h = hi;
  return __builtin_bit_cast(
      i32x8, __builtin_shufflevector(l, h, 0, 1, 2, 3, 4, 5, 6, 7));
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(64 * kNW, 2) void fwd_fp8_kernel(
    const uint8_t* __restrict__ Q8, const uint8_t* __restrict__ K8,
    const uint8_t* __restrict__ V8, uint16_t* __restrict__ O,
    float* __restrict__ LSE, int N, int Np, int n_qblk, float c_log2) {
  constexpr int RB = FA_FP8_ROW_BYTES(D);
  constexpr int KSTAGE = kBC * RB;        // bytes of a K tile
  constexpr int VSTAGE = D * kVRB;        // bytes of a V tile
  constexpr int KI = KSTAGE / 1024, VI = VSTAGE / 1024;   // 1 KB DMAs
  static_assert(KSTAGE % 1024 == 0 && VSTAGE % 1024 == 0, "DMA tiles");
  constexpr int kIW = (KI + VI + kNW - 1) / kNW;
  constexpr int kMinBatch = (KI + VI) / kNW;       // DMAs of every wave
  static_assert(kMinBatch >= 1 && 2 * kMinBatch < 16, "vmcnt range");
  constexpr int NM = D / 64;                       // S MFMAs per 32 keys
  __shared__ __attribute__((aligned(16))) uint8_t lds_k[kNS][KSTAGE];
  __shared__ __attribute__((aligned(16))) uint8_t lds_v[kNS][VSTAGE];

  const int BH = gridDim.x / n_qblk;
  int bh, qb;
  block_schedule((int)blockIdx.x, n_qblk, BH, CAUSAL, bh, qb);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = wave_id();
  const int lq = lane & 31;
  const int hh = lane >> 5;
  const int q0 = qb * kBR;
  const int qlo = q0 + 32 * w;
  const int qrow = qlo + lq;

  int kend = N;
  if (CAUSAL) kend = min(kend, q0 + kBR);
  const int ntiles = (kend + kBC - 1) / kBC;
  int kend_w = N;
  if (CAUSAL) kend_w = min(kend_w, qlo + 32);
  const int nt_w = kend_w > 0 ? (kend_w + kBC - 1) / kBC : 0;

  const uint8_t* Qh = Q8 + (size_t)bh * Np * RB;
  const uint8_t* Kh = K8 + (size_t)bh * Np * RB;
  const uint8_t* Vh = V8 + (size_t)bh * (Np / kBC) * VSTAGE;

  // Q fragment (B operand of S^T = K Q^T): query qrow (rows past N are
  // zero; rows past N are not read), coordinates [64m + 16hh, +16)
  // and [64m + 32 + 16hh, +16); scale byte m = block 2m + hh.
  i32x8 qf[NM];
  unsigned qs = kE8M0One;
#pragma unroll
  for (int m = 0; m < NM; ++m) qf[m] = i32x8{};
  if (qrow < N) {
    const uint8_t* qr = Qh + (size_t)qrow * RB;
#pragma unroll
    for (int m = 0; m < NM; ++m)
      qf[m] = join8(*(const u32x4*)(qr + 64 * m + 16 * hh),
                    *(const u32x4*)(qr + 64 * m + 32 + 16 * hh));
    qs = D == 128 ? (unsigned)*(const uint16_t*)(qr + D + 2 * hh)
                  : (unsigned)qr[D + hh];
  }
  // A negative scale flips the sign bit of every Q code (exact).
  if (c_log2 < 0.f) {
#pragma unroll
    for (int m = 0; m < NM; ++m) qf[m] ^= (int)0x80808080;
    c_log2 = -c_log2;
  }
  c_log2 = fmaxf(c_log2, 1e-30f);
  __builtin_amdgcn_s_waitcnt(kWaitVm0);

  // DMA: a tile is KI + VI transfers of 1 KB (K bytes [1024 i, +1024),
  // then V's); wavefront w issues transfers w, w + 8, ...
  const unsigned lk0 = lds_addr(&lds_k[0][0]);
  const unsigned lv0 = lds_addr(&lds_v[0][0]);
  auto dma_tile = [&](int j, int st) {
    const auto rk = byte_rsrc(Kh + (size_t)j * KSTAGE, KSTAGE);
    const auto rv = byte_rsrc(Vh + (size_t)j * VSTAGE, VSTAGE);
#pragma unroll
    for (int u = 0; u < kIW; ++u) {
      const int g = w + kNW * u;
      if (g < KI)
        lds_dma16(rk, lk0 + (unsigned)(st * KSTAGE + 1024 * g),
                  (unsigned)(1024 * g + 16 * lane));
      else if (g < KI + VI)
        lds_dma16(rv, lv0 + (unsigned)(st * VSTAGE + 1024 * (g - KI)),
                  (unsigned)(1024 * (g - KI) + 16 * lane));
    }
  };

  f32x16 oacc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) oacc[i] = f32x16{};
  float m_ref = -INFINITY, m_use = 0.f, l_run = 0.f;

  const int last = ntiles - 1;
#pragma unroll
  for (int j = 0; j < kNS - 1; ++j)
    if (j <= last) dma_tile(j, j);

  for (int j = 0; j < ntiles; ++j) {
    // Tile j's transfers were issued three tiles ago; the two younger
    // batches may stay in flight.
    if (j + 2 <= last)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * kMinBatch) : "memory");
    else if (j + 1 <= last)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kMinBatch) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (j + kNS - 1 <= last) dma_tile(j + kNS - 1, (j + kNS - 1) % kNS);
    if (j >= nt_w) continue;
    const uint8_t* ks = &lds_k[j % kNS][0];
    const uint8_t* vs = &lds_v[j % kNS][0];

    // ---- S^T = K Q^T for the two 32-key halves t (K rows 32t + lq).
    f32x16 s[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const uint8_t* kr = ks + (32 * t + lq) * RB;
      const unsigned ksc = D == 128 ? (unsigned)*(const uint16_t*)(kr + D + 2 * hh)
                                    : (unsigned)kr[D + hh];
      s[t] = f32x16{};
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const i32x8 a = join8(*(const u32x4*)(kr + 64 * m + 16 * hh),
                              *(const u32x4*)(kr + 64 * m + 32 + 16 * hh));
        if (m == 0) s[t] = mfma_fp8<0>(a, qf[0], s[t], ksc, qs);
        else s[t] = mfma_fp8<1>(a, qf[NM - 1], s[t], ksc, qs);
      }
    }

    // ---- mask: register r of half t holds key 64j + 32t + 16hh + r.
    const int k0 = j * kBC;
    const bool need_mask = (CAUSAL && k0 + kBC - 1 > qlo) || (k0 + kBC > N);
    if (need_mask) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + 32 * t + 16 * hh + r;
          if ((CAUSAL && key > qrow) || key >= N) s[t][r] = -INFINITY;
        }
    }

    // ---- weights against the reference; move it when a lane's sum would
    // exceed kSumLimit (or on the row's first tile), rescaling O and l.
    float p[2][16];
    float tsum = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        p[t][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[t][r], c_log2, -m_use));
        tsum += p[t][r];
      }
    if (__builtin_expect(__any(tsum > kSumLimit || m_ref == -INFINITY), 0)) {
      float mx = -INFINITY;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[t][r]);
      mx = max_halves(mx);
      const float mt = (mx == -INFINITY) ? -INFINITY : mx * c_log2;
      const float m_new = fmaxf(m_ref, mt);
      const float alpha =
          __builtin_amdgcn_exp2f(m_ref - ((m_new == -INFINITY) ? 0.f : m_new));
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < D / 32; ++i) oacc[i] *= alpha;
      m_ref = m_new;
      m_use = (m_new == -INFINITY) ? 0.f : m_new;
      tsum = 0.f;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          p[t][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[t][r], c_log2, -m_use));
          tsum += p[t][r];
        }
    }
    l_run += tsum;

    // ---- P^T as E4M3 (byte e = key 32(e/16) + 16hh + e%16).
    i32x8 pf;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int t = i / 4, r = 4 * (i % 4);
      pf[i] = (int)pack_fp8x4(p[t][r], p[t][r + 1], p[t][r + 2], p[t][r + 3]);
    }

    // ---- O^T += V^T P^T: V^T rows 32db + lq, keys [16hh, +16) and
    // [32 + 16hh, +16), scale byte 64 + hh.
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const uint8_t* vr = vs + (32 * db + lq) * kVRB;
      const i32x8 a = join8(*(const u32x4*)(vr + 16 * hh),
                            *(const u32x4*)(vr + 32 + 16 * hh));
      oacc[db] = mfma_fp8<0>(a, pf, oacc[db], (unsigned)vr[64 + hh], kE8M0One);
    }
  }

  // ---- epilogue: O = acc / l (bf16), LSE = (m_ref + log2 l) ln 2.
  const float l_tot = sum_halves(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (qrow < N) {
    uint16_t* orow = O + ((size_t)bh * N + qrow) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = oacc[db][4 * g + e] * inv;
        *(bf16x4*)(orow + 32 * db + 8 * g + 4 * hh) = to_bf16x4(x);
      }
    }
    if (hh == 0)
      LSE[(size_t)bh * N + qrow] =
          l_tot > 0.f ? (m_ref + __builtin_amdgcn_logf(l_tot)) * kLn2 : -INFINITY;
  }
}

}  // namespace

int launch_fp8_quantize(const uint16_t* q, const uint16_t* k,
                        const uint16_t* v, const int8_t* signs, uint8_t* ws,
                        int B, int H, int N, int d, hipStream_t stream) {
  const long long BH = (long long)B * H;
  const int Np = (N + kBC - 1) / kBC * kBC;
  const int RB = FA_FP8_ROW_BYTES(d);
  const long long rows = BH * Np;
  uint8_t* q8 = ws;
  uint8_t* k8 = ws + (size_t)rows * RB;
  uint8_t* v8 = ws + 2 * (size_t)rows * RB;
  const int rpb = kQThreads / (d / 32);
  const int tpw = kQThreads / (2 * d);
  const int nrb = (int)((rows + rpb - 1) / rpb);
  const int nvb = (int)((rows / kBC + tpw - 1) / tpw);
  const dim3 grid((unsigned)(2 * nrb + nvb)), block(kQThreads);
  if (d == 128)
    hipLaunchKernelGGL((fp8_quant_kernel<128>), grid, block, 0, stream, q, k,
                       v, signs, q8, k8, v8, N, Np, rows, nrb);
  else
    hipLaunchKernelGGL((fp8_quant_kernel<64>), grid, block, 0, stream, q, k,
                       v, signs, q8, k8, v8, N, Np, rows, nrb);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

int launch_fwd_fp8(const uint8_t* ws, uint16_t* o, float* lse, int B, int H,
                   int N, int d, float score_scale, int causal,
                   hipStream_t stream) {
  const long long BH = (long long)B * H;
  const int Np = (N + kBC - 1) / kBC * kBC;
  const int RB = FA_FP8_ROW_BYTES(d);
  const long long rows = BH * Np;
  const uint8_t* q8 = ws;
  const uint8_t* k8 = ws + (size_t)rows * RB;
  const uint8_t* v8 = ws + 2 * (size_t)rows * RB;
  const int n_qblk = (N + kBR - 1) / kBR;
  const dim3 grid((unsigned)(BH * n_qblk)), block(64 * kNW);
  const float c = (float)((double)score_scale * 1.4426950408889634);
#define FA_FP8_LAUNCH(DD, CC)                                              \
  hipLaunchKernelGGL((fwd_fp8_kernel<DD, CC>), grid, block, 0, stream, q8, \
                     k8, v8, o, lse, N, Np, n_qblk, c)
  if (d == 128) {
    if (causal) FA_FP8_LAUNCH(128, true); else FA_FP8_LAUNCH(128, false);
  } else {
    if (causal) FA_FP8_LAUNCH(64, true); else FA_FP8_LAUNCH(64, false);
  }
#undef FA_FP8_LAUNCH
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // namespace fa
