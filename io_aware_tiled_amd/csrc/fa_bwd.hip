// Backward kernels of libfa: gradients of exact attention with P recomputed
// tile by tile from the stored log-sum-exp.
//
// Pages cited (titles as the pages give them):
//   [MM] "Is a full-day context better than a 10-minute context? Flash
//        attention and the sequence-length question" (marketmaker.cc blog)
//   [TW] "Flash-Attention 2 for performance optimisation" (Medium blog)
//   [ZN] "Paper summary: FlashAttention" (zenn.dev)
//
// The forward keeps only O and the per-row statistic; the backward
// recomputes each score tile from Q and K and turns it back into
// probabilities with that statistic instead of reading a stored N x N matrix
// ([MM] "Backward pass: recompute instead of store"; [TW] "Recomputation";
// [ZN] "Proposed method").  With the natural-log LSE of the forward,
// P = exp(scale * Q K^T - LSE) needs no running maximum.  The gradient is
// that of <dO, O>:
//   dV = P^T dO,  dP = dO V^T,  D_i = dO_i . O_i,  dS = P * (dP - D),
//   dQ = scale dS K,  dK = scale dS^T Q.
//
// Kernels (three launches on one stream):
//   1. bwd_preprocess: D_i from the bf16 O and dO, and zero the float32 dQ
//      accumulator.
//   2. bwd_dkdv: one workgroup per (batch, head, 128-key block); 4
//      wavefronts own 32 keys each and walk the 32-row query tiles that can
//      see those keys (causal: tiles wholly before the key block are
//      skipped).  dK and dV accumulate in registers; dQ is accumulated with
//      float32 atomic adds.
//   3. bwd_dq_convert: dQ accumulator * scale -> bf16.
//
// gfx950 mapping in bwd_dkdv (head dim 128):
//   * S = Q_i K_j^T and dP = dO_i V_j^T on v_mfma_f32_32x32x16_bf16 with
//     K_j / V_j as register-resident B operands; the accumulator layout puts
//     one key per lane and 16 queries per lane, so P and dS are directly the
//     B operands of dV^T += dO_i^T P and dK^T += Q_i^T dS.
//   * dO_i^T and Q_i^T come from the row-major LDS tiles through
//     ds_read_b64_tr_b16; Q_i, dO_i and K_j use a 16-byte-chunk XOR swizzle
//     that keeps both the row reads (ds_read_b128) and the transposed reads
//     free of bank conflicts.
//   * dS^T goes to LDS with 8-byte stores; dQ_i += dS K_j reads it back
//     transposed (ds_read_b64_tr_b16), each wavefront producing 32 columns
//     of dQ over all 128 keys.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

namespace {

constexpr int kThreads = 256;
constexpr int kBK = 128;   // keys per workgroup (32 per wavefront)
constexpr int kBQ = 32;    // query rows per tile
constexpr int kD = 128;    // head dimension of the backward kernel

// 16-byte chunk swizzle of a 256-byte row: rows 0..15 at one chunk land in
// 16 distinct chunks, and rows 4a..4a+3 map any aligned group of 4 chunks to
// 4 distinct groups.
__device__ __forceinline__ int swz(int row) {
  return ((row & 3) << 2) | ((row >> 2) & 3);
}
// Element offset of (row, col) in a swizzled [rows][128] bf16 tile.
__device__ __forceinline__ int sw_off(int row, int col) {
  return row * kD + ((((col >> 3) ^ swz(row)) << 3) | (col & 7));
}

// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_preprocess_kernel(
    const uint16_t* __restrict__ O, const uint16_t* __restrict__ dO,
    float* __restrict__ Dv, float* __restrict__ dq_acc, size_t rows) {
  constexpr int TPR = D / 8;                 // threads per row
  constexpr int RPB = kThreads / TPR;        // rows per block
  const int t = threadIdx.x % TPR;
  const size_t row = (size_t)blockIdx.x * RPB + threadIdx.x / TPR;
  float acc = 0.f;
  if (row < rows) {
    const bf16x8 o = *(const bf16x8*)(O + row * D + 8 * t);
    const bf16x8 g = *(const bf16x8*)(dO + row * D + 8 * t);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += (float)o[e] * (float)g[e];
    f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
    *(f32x4*)(dq_acc + row * D + 8 * t) = z;
    *(f32x4*)(dq_acc + row * D + 8 * t + 4) = z;
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (row < rows && t == 0) Dv[row] = acc;
}

__global__ __launch_bounds__(kThreads) void bwd_dq_convert_kernel(
    const float* __restrict__ acc, uint16_t* __restrict__ dq, size_t n8,
    float scale) {
  const size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= n8) return;
  f32x8 x;
  const f32x4 a = *(const f32x4*)(acc + 8 * i);
  const f32x4 b = *(const f32x4*)(acc + 8 * i + 4);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[e] = a[e] * scale;
    x[e + 4] = b[e] * scale;
  }
  *(bf16x8*)(dq + 8 * i) = to_bf16x8(x);
}

// ---------------------------------------------------------------------------
template <bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void bwd_dkdv_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
    const float* __restrict__ LSE, const float* __restrict__ Dv,
    float* __restrict__ dq_acc, uint16_t* __restrict__ dK,
    uint16_t* __restrict__ dV, int N, int n_kblk, float c_log2,
    float scale) {
  constexpr int D = kD;
  __shared__ __attribute__((aligned(16))) uint16_t lds_k[kBK * D];     // 32 KB
  __shared__ __attribute__((aligned(16))) uint16_t lds_q[kBQ * D];     //  8 KB
  __shared__ __attribute__((aligned(16))) uint16_t lds_do[kBQ * D];    //  8 KB
  __shared__ __attribute__((aligned(16))) uint16_t lds_dst[kBK * kBQ]; //  8 KB
  __shared__ __attribute__((aligned(16))) float lds_lse[kBQ];
  __shared__ __attribute__((aligned(16))) float lds_d[kBQ];

  const int BH = gridDim.x / n_kblk;
  // Key blocks with the most visible queries (smallest index) go first.
  const int jb = blockIdx.x / BH;
  const int bh = blockIdx.x % BH;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int r16 = lane & 15;
  const int dsub = (lane >> 4) & 1;

  const int kb0 = jb * kBK;
  const int mykey = kb0 + 32 * w + l32;      // this lane's key
  const size_t head = (size_t)bh * N * D;
  const uint16_t* Qh = Q + head;
  const uint16_t* Kh = K + head;
  const uint16_t* Vh = V + head;
  const uint16_t* dOh = dO + head;
  const float* LSEh = LSE + (size_t)bh * N;
  const float* Dh = Dv + (size_t)bh * N;
  float* dQh = dq_acc + head;

  // ---- K_j into LDS (swizzled), K_j and V_j fragments into registers.
#pragma unroll
  for (int r = 0; r < kBK * D / 8 / kThreads; ++r) {
    const int c = tid + kThreads * r;
    const int row = c / (D / 8);
    const int col = 8 * (c % (D / 8));
    const int key = kb0 + row;
    u32x4 x = u32x4{0, 0, 0, 0};
    if (key < N) x = *(const u32x4*)(Kh + (size_t)key * D + col);
    *(u32x4*)(&lds_k[sw_off(row, col)]) = x;
  }
  bf16x8 kf[D / 16], vf[D / 16];   // lane: key mykey, d = 16kk + 8hh + 0..7
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    if (mykey < N) {
      kf[kk] = *(const bf16x8*)(Kh + (size_t)mykey * D + 16 * kk + 8 * hh);
      vf[kk] = *(const bf16x8*)(Vh + (size_t)mykey * D + 16 * kk + 8 * hh);
    } else {
      kf[kk] = bf16x8{};
      vf[kk] = bf16x8{};
    }
  }

  f32x16 dk_acc[D / 32], dv_acc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) {
    dk_acc[i] = f32x16{};
    dv_acc[i] = f32x16{};
  }

  const int n_qt = (N + kBQ - 1) / kBQ;
  const int it0 = CAUSAL ? kb0 / kBQ : 0;

  // Query-tile staging: 2 chunks of Q and 2 of dO per thread, plus LSE / D.
  u32x4 qreg[2], doreg[2];
  float lse_r = 0.f, d_r = 0.f;
  auto load_qtile = [&](int it) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int c = tid + kThreads * r;
      const int row = c / (D / 8);
      const int col = 8 * (c % (D / 8));
      const int q = it * kBQ + row;
      if (q < N) {
        qreg[r] = *(const u32x4*)(Qh + (size_t)q * D + col);
        doreg[r] = *(const u32x4*)(dOh + (size_t)q * D + col);
      } else {
        qreg[r] = u32x4{0, 0, 0, 0};
        doreg[r] = u32x4{0, 0, 0, 0};
      }
    }
    if (tid < kBQ) {
      const int q = it * kBQ + tid;
      // Rows past N (and rows without any visible key) get +inf so that
      // exp2(s - lse) = 0 for every key.
      float l = q < N ? LSEh[q] : INFINITY;
      lse_r = (l == -INFINITY) ? INFINITY : l * kLog2e;
      d_r = q < N ? Dh[q] : 0.f;
    }
  };
  auto store_qtile = [&]() {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int c = tid + kThreads * r;
      const int row = c / (D / 8);
      const int col = 8 * (c % (D / 8));
      *(u32x4*)(&lds_q[sw_off(row, col)]) = qreg[r];
      *(u32x4*)(&lds_do[sw_off(row, col)]) = doreg[r];
    }
    if (tid < kBQ) {
      lds_lse[tid] = lse_r;
      lds_d[tid] = d_r;
    }
  };

  if (it0 < n_qt) load_qtile(it0);
  for (int it = it0; it < n_qt; ++it) {
    store_qtile();
    __syncthreads();                      // (A) Q_i, dO_i, LSE, D, K ready
    if (it + 1 < n_qt) load_qtile(it + 1);

    const int q0 = it * kBQ;
    const int wk0 = kb0 + 32 * w;        // first key of this wavefront
    const bool active = !(CAUSAL && wk0 > q0 + kBQ - 1) && wk0 < N;

    bf16x8 dsb[2];
    if (active) {
      // ---- S = Q_i K_j^T and dP = dO_i V_j^T (queries x keys).
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const int off = sw_off(l32, 16 * kk + 8 * hh);
        const bf16x8 qa = *(const bf16x8*)(&lds_q[off]);
        const bf16x8 ga = *(const bf16x8*)(&lds_do[off]);
        s = mfma32x16(qa, kf[kk], s);
        dp = mfma32x16(ga, vf[kk], dp);
      }
      // ---- P = exp2(s*c - lse2), dS = P (dP - D).  Register r holds query
      // q0 + 8(r/4) + 4hh + r%4 of this lane's key.
      const bool need_mask =
          (CAUSAL && wk0 + 31 > q0) || (wk0 + 32 > N);
      f32x8 pv[2], dsv[2];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 l4 = *(const f32x4*)(&lds_lse[8 * g + 4 * hh]);
        const f32x4 d4 = *(const f32x4*)(&lds_d[8 * g + 4 * hh]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g + e;
          float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c_log2, -l4[e]));
          if (need_mask) {
            const int q = q0 + 8 * g + 4 * hh + e;
            if ((CAUSAL && mykey > q) || mykey >= N) p = 0.f;
          }
          const float ds = p * (dp[r] - d4[e]);
          pv[r >> 3][r & 7] = p;
          dsv[r >> 3][r & 7] = ds;
        }
      }
      const bf16x8 pb[2] = {to_bf16x8(pv[0]), to_bf16x8(pv[1])};
      dsb[0] = to_bf16x8(dsv[0]);
      dsb[1] = to_bf16x8(dsv[1]);

      // ---- dV^T += dO_i^T P and dK^T += Q_i^T dS (d x keys).
      // Operand slot (hh, e) <-> query 16c + 8(e/4) + 4hh + e%4.
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const int col = 32 * db + 16 * dsub + 4 * (r16 & 3);
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const int row = 16 * c + 4 * hh + (r16 >> 2);
          const i16x4 g_lo = lds_read_tr16(&lds_do[sw_off(row, col)]);
          const i16x4 g_hi = lds_read_tr16(&lds_do[sw_off(row + 8, col)]);
          const i16x4 q_lo = lds_read_tr16(&lds_q[sw_off(row, col)]);
          const i16x4 q_hi = lds_read_tr16(&lds_q[sw_off(row + 8, col)]);
          dv_acc[db] = mfma32x16(join_bf16(g_lo, g_hi), pb[c], dv_acc[db]);
          dk_acc[db] = mfma32x16(join_bf16(q_lo, q_hi), dsb[c], dk_acc[db]);
        }
      }
    } else {
      dsb[0] = bf16x8{};
      dsb[1] = bf16x8{};
    }

    // ---- dS^T to LDS: row = key (32w + l32), 4 consecutive queries per store.
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const bf16x4 x = (g & 1) ? hi4(dsb[g >> 1]) : lo4(dsb[g >> 1]);
      *(bf16x4*)(&lds_dst[(32 * w + l32) * kBQ + 8 * g + 4 * hh]) = x;
    }
    __syncthreads();                      // (B) dS^T complete

    // ---- dQ_i[:, 32w .. 32w+31] += dS K_j over the 128 keys.
    // Slot (hh, e) <-> key 16kc + 8(e/4) + 4hh + e%4 for both operands.
    if (!(CAUSAL && kb0 > q0 + kBQ - 1)) {
      f32x16 dq = f32x16{};
      const int qcol = 16 * dsub + 4 * (r16 & 3);
      const int dcol = 32 * w + 16 * dsub + 4 * (r16 & 3);
#pragma unroll
      for (int kc = 0; kc < kBK / 16; ++kc) {
        const int krow = 16 * kc + 4 * hh + (r16 >> 2);
        const i16x4 a_lo = lds_read_tr16(&lds_dst[krow * kBQ + qcol]);
        const i16x4 a_hi = lds_read_tr16(&lds_dst[(krow + 8) * kBQ + qcol]);
        const i16x4 b_lo = lds_read_tr16(&lds_k[sw_off(krow, dcol)]);
        const i16x4 b_hi = lds_read_tr16(&lds_k[sw_off(krow + 8, dcol)]);
        dq = mfma32x16(join_bf16(a_lo, a_hi), join_bf16(b_lo, b_hi), dq);
      }
      // Register r holds query q0 + 8(r/4) + 4hh + r%4, column 32w + l32.
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int q = q0 + 8 * (r / 4) + 4 * hh + (r % 4);
        if (q < N) unsafeAtomicAdd(&dQh[(size_t)q * D + 32 * w + l32], dq[r]);
      }
    }
  }

  // ---- epilogue: dK = scale * dK^T, dV = dV^T (lane = key, regs = d).
  if (mykey < N) {
    uint16_t* dkr = dK + head + (size_t)mykey * D;
    uint16_t* dvr = dV + head + (size_t)mykey * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 a, b;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a[e] = dk_acc[db][4 * g + e] * scale;
          b[e] = dv_acc[db][4 * g + e];
        }
        *(bf16x4*)(dkr + 32 * db + 8 * g + 4 * hh) = to_bf16x4(a);
        *(bf16x4*)(dvr + 32 * db + 8 * g + 4 * hh) = to_bf16x4(b);
      }
    }
  }
}

}  // namespace

int launch_bwd_preprocess(const uint16_t* o, const uint16_t* dO, float* D,
                          float* dq_acc, int B, int H, int N, int d,
                          hipStream_t stream) {
  const size_t rows = (size_t)B * H * N;
  if (d == 128) {
    constexpr int RPB = kThreads / (128 / 8);
    const dim3 grid((unsigned)((rows + RPB - 1) / RPB));
    hipLaunchKernelGGL(bwd_preprocess_kernel<128>, grid, dim3(kThreads), 0,
                       stream, o, dO, D, dq_acc, rows);
  } else {
    constexpr int RPB = kThreads / (64 / 8);
    const dim3 grid((unsigned)((rows + RPB - 1) / RPB));
    hipLaunchKernelGGL(bwd_preprocess_kernel<64>, grid, dim3(kThreads), 0,
                       stream, o, dO, D, dq_acc, rows);
  }
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

int launch_bwd_dkdv(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                    const uint16_t* dO, const float* lse, const float* D,
                    float* dq_acc, uint16_t* dk, uint16_t* dv, int B, int H,
                    int N, int d, float scale, int causal,
                    hipStream_t stream) {
  if (d != kD) return -3;
  const int n_kblk = (N + kBK - 1) / kBK;
  const dim3 grid((unsigned)(B * H * n_kblk)), block(kThreads);
  const float c = (float)((double)scale * 1.4426950408889634);
  if (causal) {
    hipLaunchKernelGGL(bwd_dkdv_kernel<true>, grid, block, 0, stream, q, k, v,
                       dO, lse, D, dq_acc, dk, dv, N, n_kblk, c, scale);
  } else {
    hipLaunchKernelGGL(bwd_dkdv_kernel<false>, grid, block, 0, stream, q, k,
                       v, dO, lse, D, dq_acc, dk, dv, N, n_kblk, c, scale);
  }
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

int launch_bwd_dq_convert(const float* dq_acc, uint16_t* dq, size_t n,
                          float scale, hipStream_t stream) {
  const size_t n8 = n / 8;
  const dim3 grid((unsigned)((n8 + kThreads - 1) / kThreads));
  hipLaunchKernelGGL(bwd_dq_convert_kernel, grid, dim3(kThreads), 0, stream,
                     dq_acc, dq, n8, scale);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // namespace fa
