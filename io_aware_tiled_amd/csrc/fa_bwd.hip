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
// Kernels (three launches on one stream, no atomics, deterministic):
//   1. bwd_preprocess: D_i = dO_i . O_i from the bf16 O and dO.
//   2. dK/dV: one workgroup per (batch, head, 128-key block) that visits
//      every 64-row query tile that can see its keys (causal: tiles wholly
//      before the key block are skipped); S, dP, P and dS are recomputed
//      per tile and dK^T, dV^T accumulate in registers.
//        bwd_dkdv_pipe_kernel (grids that fill the chip): 4 wavefronts of
//        32 keys, K and V fragments held in registers, dK/dV accumulators
//        in AGPRs, query tiles by LDS DMA through four stages, two
//        software-pipelined phases per tile; one workgroup per CU at head
//        dim 128, two at head dim 64 (fewer registers, smaller tiles).
//        bwd_dkdv_kernel (small grids without a block mask, and head dim 64
//        with dropout): 8 wavefronts, each owning 32 keys and one half of
//        every query tile; the two halves' partials are added through LDS
//        at the end.
//   3. dQ: streams K/V tiles like the forward, recomputes S^T and dP^T and
//      accumulates dQ^T in registers.
//        bwd_dq_pipe_kernel (grids that fill the chip): 256-row query
//        blocks, 8 wavefronts of 32 rows, K/V by LDS DMA through four
//        stages, software-pipelined over 32-key half-tiles.
//        bwd_dq_kernel (small grids without a block mask, and head dim 64
//        with dropout): 128-row query blocks, 4 wavefronts, register-staged
//        double buffer.
// Splitting dQ from dK/dV costs 4d extra matrix FLOP per (query, key) pair
// (14d instead of 10d) but removes the float32 atomics that a fused kernel
// needs for dQ: device-scope atomics are resolved at the memory side, not in
// an XCD's L2, and on gfx950 they cost more than the recomputation.
//
// gfx950 mapping (head dim 128):
//   * bwd_dkdv computes S = Q_i K_j^T and dP = dO_i V_j^T on
//     v_mfma_f32_32x32x16_bf16 so the accumulator puts one key per lane and
//     16 queries per lane; P and dS are then directly the B operands of
//     dV^T += dO_i^T P and dK^T += Q_i^T dS, with dO_i^T and Q_i^T read from
//     the row-major LDS tiles by ds_read_b64_tr_b16.
//   * bwd_dq computes S^T and dP^T with one query per lane (as the forward),
//     so P^T and dS^T need only the lane's own LSE and D, and dS^T is the B
//     operand of dQ^T += K_j^T dS^T with K_j^T read transposed from LDS.
//   * The pipelined kernels' streamed tiles sit in LDS rows padded to 272
//     bytes, placed by tile_slot so that both the 16-byte row reads and the
//     transposed reads are free of bank conflicts; the small-grid kernels
//     pad rows to 304 bytes (conflict-free row reads, at most 2-way
//     transposed reads).
#include "fa.h"
#include "fa_common.h"
#include "fa_launch.h"

#include <type_traits>

namespace fa {

namespace {

constexpr int kThreads = 256;
constexpr int kBK = 128;   // keys per workgroup (32 per wavefront)
// Block-sparse backward: query and key tiles of one head are listed in LDS
// as 16-bit entries, at most this many (64-row tiles up to N = 131072).
constexpr int kSparseMaxTiles = 2 * FA_SPARSE_MAX_KEY_BLOCKS;
static_assert(FA_SPARSE_BK == kBK, "a block-mask column is one dK/dV workgroup");
constexpr int kD = 128;    // head dimension of the pipelined backward kernels

// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_preprocess_kernel(
    const uint16_t* __restrict__ O, const uint16_t* __restrict__ dO,
    float* __restrict__ Dv, size_t rows) {
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
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (row < rows && t == 0) Dv[row] = acc;
}

// ---------------------------------------------------------------------------
// dK/dV kernel: 8 wavefronts (two per SIMD).  Wavefront w owns the 32 keys
// of key slice ks = w % 4 and the 32 query rows of half qh = w / 4 of each
// 64-row query tile, so wave pairs (ks, 0) and (ks, 1) hold partial dK/dV of
// the same keys and add them through LDS once at the end.
constexpr int kBwdThreads = 512;
constexpr int kBQ2 = 64;   // query rows per tile

// Padded row stride (elements) of the small-grid kernels: 304-byte rows for
// the 256-byte K/V/Q/dO rows keep the 16-byte row reads conflict-free and the
// transposed 8-byte reads at most 2-way.  Linear layouts let every operand
// address be one per-lane base plus an immediate offset.
constexpr int kRS = 152;   // K, V, Q, dO row stride

template <int D, bool CAUSAL, bool DROP = false, bool SPARSE = false>
__global__ __launch_bounds__(kBwdThreads, 1) void bwd_dkdv_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
    const float* __restrict__ LSE, const float* __restrict__ Dv,
    uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int N, int n_kblk,
    float c_log2, float scale, Dropout drop, const uint8_t* __restrict__ bmask,
    int H, const int32_t* __restrict__ kv_len = nullptr) {
  static_assert(D == 64 || D == 128, "head dimension");
  constexpr int KB = kBK * kRS;        // elements of the K (or V) block
  constexpr int QB = kBQ2 * kRS;       // elements of a Q (or dO) tile
  // K | V | Q0 | dO0 | Q1 | dO1 (bf16), then LSE and D (float), the query
  // tiles double-buffered so one barrier per tile suffices.  After the main
  // loop the K|V region (64 KB) is reused for the dK/dV pair reduction.
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * KB + 4 * QB];
  __shared__ __attribute__((aligned(16))) float lds_lse[2][kBQ2];
  __shared__ __attribute__((aligned(16))) float lds_d[2][kBQ2];
  // Tile bases are opaque scalars: ds_read/ds_write immediate offsets are
  // 16-bit, so with bases folded in as constants every operand address of a
  // tile past 64 KB would need its own register.
  uint16_t* lds_k = smem;
  uint16_t* lds_v = smem + __builtin_amdgcn_readfirstlane(KB);
  uint16_t* const lds_q0 = smem + __builtin_amdgcn_readfirstlane(2 * KB);
  const int qbuf = __builtin_amdgcn_readfirstlane(2 * QB);   // buffer stride
  const int dooff = __builtin_amdgcn_readfirstlane(QB);      // Q -> dO
  float* red = (float*)smem;

  const int BH = gridDim.x / n_kblk;
  // Key blocks with the most visible queries (smallest index) go first.
  const int jb = blockIdx.x / BH;
  const int bh = blockIdx.x % BH;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = wave_id();   // wave-uniform (scalar register)
  const int ks = w & 3;          // key slice
  const int qh = w >> 2;         // query half of each tile
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int r16 = lane & 15;
  const int dsub = (lane >> 4) & 1;

  const int kb0 = jb * kBK;
  const int wk0 = kb0 + 32 * ks;            // first key of this wavefront
  const int mykey = wk0 + l32;              // this lane's key
  const size_t head = (size_t)bh * N * D;
  const uint16_t* Qh = Q + head;
  const uint16_t* Kh = K + head;
  const uint16_t* Vh = V + head;
  const uint16_t* dOh = dO + head;
  const float* LSEh = LSE + (size_t)bh * N;
  const float* Dh = Dv + (size_t)bh * N;

  // ---- K_j and V_j into LDS (padded rows), rows past N are zero.
#pragma unroll
  for (int r = 0; r < kBK * D / 8 / kBwdThreads; ++r) {
    const int c = tid + kBwdThreads * r;
    const int row = c / (D / 8);
    const int col = 8 * (c % (D / 8));
    const int key = kb0 + row;
    u32x4 xk = u32x4{0, 0, 0, 0}, xv = u32x4{0, 0, 0, 0};
    if (key < N) {
      xk = *(const u32x4*)(Kh + (size_t)key * D + col);
      xv = *(const u32x4*)(Vh + (size_t)key * D + col);
    }
    *(u32x4*)(&lds_k[row * kRS + col]) = xk;
    *(u32x4*)(&lds_v[row * kRS + col]) = xv;
  }

  f32x16 dk_acc[D / 32], dv_acc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) {
    dk_acc[i] = f32x16{};
    dv_acc[i] = f32x16{};
  }

  const int n_qt = (N + kBQ2 - 1) / kBQ2;
  // Key padding: keys >= kv_len[b] are masked (a block wholly past it
  // visits no query tile and writes dK = dV = 0).
  const int kvlim = kv_len ? min(max(kv_len[bh / H], 0), N) : N;
  const int it0 = CAUSAL ? kb0 / kBQ2 : 0;

  // Query tiles to visit: it0 .. n_qt - 1, or (block-sparse: the 128 keys
  // are one block-mask column) the 64-row tiles whose block row keeps the
  // column, listed in LDS.
  __shared__ uint16_t qt_list[SPARSE ? kSparseMaxTiles : 1];
  __shared__ int qt_count;
  int n_vis = n_qt - it0;
  if constexpr (SPARSE) {
    const int n_mk = (N + FA_SPARSE_BK - 1) / FA_SPARSE_BK;
    const int n_mq = (N + FA_SPARSE_BQ - 1) / FA_SPARSE_BQ;
    const uint8_t* mcol = bmask + (size_t)(bh % H) * n_mq * n_mk + jb;
    if (w == 0) {
      int cnt = 0;
      for (int base = it0; base < n_qt; base += 64) {
        const int q = base + lane;
        const bool keep =
            q < n_qt && mcol[(size_t)(q * kBQ2 / FA_SPARSE_BQ) * n_mk] != 0;
        const unsigned long long bal = __ballot(keep);
        const int below = __builtin_popcountll(bal & ((1ull << lane) - 1ull));
        if (keep) qt_list[cnt + below] = (uint16_t)q;
        cnt += __builtin_popcountll(bal);
      }
      if (lane == 0) qt_count = cnt;
    }
    __syncthreads();
    n_vis = qt_count;
  }
  if (kb0 >= kvlim) n_vis = 0;
  auto qtile = [&](int i) -> int {
    if constexpr (SPARSE)
      return (int)__builtin_amdgcn_readfirstlane((unsigned)qt_list[i]);
    else
      return it0 + i;
  };


  // Query-tile staging: QCH 16-byte chunks of Q and of dO per thread, plus
  // LSE / D.  Rows past N load row N-1 (in bounds) and are replaced by zeros
  // with a select, so the loads need no branch.
  constexpr int QCH = kBQ2 * D / 8 / kBwdThreads;
  static_assert(QCH * 8 * kBwdThreads == kBQ2 * D, "tile staging");
  u32x4 qreg[QCH], doreg[QCH];
  float lse_r = 0.f, d_r = 0.f;
  auto load_qtile = [&](int it) {
    const int qt0 = it * kBQ2;
    const uint16_t* qb = Qh + (size_t)qt0 * D;      // wave-uniform bases
    const uint16_t* gb = dOh + (size_t)qt0 * D;
#pragma unroll
    for (int r = 0; r < QCH; ++r) {
      const int c = tid + kBwdThreads * r;
      const int row = c / (D / 8);
      const int col = 8 * (c % (D / 8));
      const bool ok = qt0 + row < N;
      const unsigned off = (unsigned)(min(row, N - 1 - qt0) * D + col);
      const u32x4 a = *(const u32x4*)(qb + off);
      const u32x4 g = *(const u32x4*)(gb + off);
      const u32x4 z = u32x4{0, 0, 0, 0};
      qreg[r] = ok ? a : z;
      doreg[r] = ok ? g : z;
    }
    if (w == 0) {
      const int q = qt0 + lane;
      const int qc = min(q, N - 1);
      // Rows past N (and rows without any visible key) get +inf so that
      // exp2(s - lse) = 0 for every key.
      const float l = q < N ? LSEh[qc] : INFINITY;
      lse_r = (l == -INFINITY) ? INFINITY : l * kLog2e;
      d_r = q < N ? Dh[qc] : 0.f;
    }
  };
  auto store_qtile = [&](int buf) {
    uint16_t* lq_ = lds_q0 + (buf ? qbuf : 0);
    uint16_t* ld_ = lq_ + dooff;
#pragma unroll
    for (int r = 0; r < QCH; ++r) {
      const int c = tid + kBwdThreads * r;
      const int row = c / (D / 8);
      const int col = 8 * (c % (D / 8));
      *(u32x4*)(&lq_[row * kRS + col]) = qreg[r];
      *(u32x4*)(&ld_[row * kRS + col]) = doreg[r];
    }
    if (w == 0) {
      lds_lse[buf][lane] = lse_r;
      lds_d[buf][lane] = d_r;
    }
  };

  if (n_vis > 0) load_qtile(qtile(0));
  for (int i = 0; i < n_vis; ++i) {
    const int it = qtile(i);
    const int buf = i & 1;
    store_qtile(buf);
    // Q_i, dO_i, LSE, D (and K, V) ready; also every wavefront has finished
    // reading the other buffer, which the next iteration overwrites.
    __syncthreads();
    if (i + 1 < n_vis) load_qtile(qtile(i + 1));
    const uint16_t* lds_q = lds_q0 + (buf ? qbuf : 0);
    const uint16_t* lds_do = lds_q + dooff;
    const float* lse_t = lds_lse[buf];
    const float* d_t = lds_d[buf];

    const int q0 = it * kBQ2;
    const int qw0 = q0 + 32 * qh;         // first query row of this wavefront

    // ---- S = Q K^T and dP = dO V^T for 32 queries x 32 keys.  (A block
    // wholly in the causal future only occurs on the diagonal tile; it is
    // computed and masked to zero rather than branched around.)
    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      const int qo = (32 * qh + l32) * kRS + 16 * kk + 8 * hh;
      const int ko = (32 * ks + l32) * kRS + 16 * kk + 8 * hh;
      const bf16x8 qa = *(const bf16x8*)(&lds_q[qo]);
      const bf16x8 ga = *(const bf16x8*)(&lds_do[qo]);
      const bf16x8 kf = *(const bf16x8*)(&lds_k[ko]);
      const bf16x8 vf = *(const bf16x8*)(&lds_v[ko]);
      s = mfma32x16(qa, kf, s);
      dp = mfma32x16(ga, vf, dp);
    }
    // ---- P = exp2(s*c - lse2), dS = P (dP - D).  Register r holds query
    // qw0 + 8(r/4) + 4hh + r%4 of this lane's key.
    const bool need_mask = (CAUSAL && wk0 + 31 > qw0) || (wk0 + 32 > kvlim);
    // Dropout: kz[g] holds the keep bytes of rows qw0 + 8g + 4hh + e (byte
    // e) for this lane's key: quad lane w makes the generator call of row
    // group w, transposes its bytes to key-major order, and the quad
    // exchange hands each lane its key's word of every call.  With Z the
    // mask and k the keep probability, dV takes P Z (1/k at the end) and
    // dS = P (Z dP / k - D).
    uint32_t kz[4];
    const float ik = DROP ? 256.f / (float)(256 - drop.p8) : 1.f;
    if constexpr (DROP) {
      kz[0] = (uint32_t)(mykey >> 2);
      kz[1] = (uint32_t)((qw0 >> 2) + 2 * (l32 & 3) + hh);
      kz[2] = (uint32_t)bh;
      kz[3] = drop.offset;
#pragma unroll
      for (int r = 0; r < 10; ++r) philox_round(kz, drop.k0, drop.k1, r);
      byte_transpose(kz);
      quad_gather(kz);
    }
    bf16x8 pb[2], dsb[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      f32x8 pv, dsv;
#pragma unroll
      for (int g2 = 0; g2 < 2; ++g2) {
        const int g = 2 * c + g2;
        const f32x4 l4 = *(const f32x4*)(&lse_t[32 * qh + 8 * g + 4 * hh]);
        const f32x4 d4 = *(const f32x4*)(&d_t[32 * qh + 8 * g + 4 * hh]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g + e;
          float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c_log2, -l4[e]));
          if (need_mask) {
            const int q = qw0 + 8 * g + 4 * hh + e;
            if ((CAUSAL && mykey > q) || mykey >= kvlim) p = 0.f;
          }
          if constexpr (DROP) {
            const bool kept = drop_keep(kz[g], e, drop.p8);
            pv[4 * g2 + e] = kept ? p : 0.f;
            dsv[4 * g2 + e] = p * ((kept ? dp[r] * ik : 0.f) - d4[e]);
          } else {
            pv[4 * g2 + e] = p;
            dsv[4 * g2 + e] = p * (dp[r] - d4[e]);
          }
        }
      }
      pb[c] = to_bf16x8(pv);
      dsb[c] = to_bf16x8(dsv);
    }

    // ---- dV^T += dO^T P and dK^T += Q^T dS (d x keys).
    // Operand slot (hh, e) <-> query row 32qh + 16c + 8(e/4) + 4hh + e%4.
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int col = 32 * db + 16 * dsub + 4 * (r16 & 3);
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int row = 32 * qh + 16 * c + 4 * hh + (r16 >> 2);
        const i16x4 g_lo = lds_read_tr16(&lds_do[row * kRS + col]);
        const i16x4 g_hi = lds_read_tr16(&lds_do[(row + 8) * kRS + col]);
        dv_acc[db] = mfma32x16(join_bf16(g_lo, g_hi), pb[c], dv_acc[db]);
      }
    }
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int col = 32 * db + 16 * dsub + 4 * (r16 & 3);
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int row = 32 * qh + 16 * c + 4 * hh + (r16 >> 2);
        const i16x4 q_lo = lds_read_tr16(&lds_q[row * kRS + col]);
        const i16x4 q_hi = lds_read_tr16(&lds_q[(row + 8) * kRS + col]);
        dk_acc[db] = mfma32x16(join_bf16(q_lo, q_hi), dsb[c], dk_acc[db]);
      }
    }

  }

  // ---- add the two query halves' partial dK^T, dV^T through LDS.
  __syncthreads();                        // K/V region free
  auto red_idx = [&](int db, int r) { return ((ks * 4 + db) * 16 + r) * 64 + lane; };
  if (qh == 1) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) red[red_idx(db, r)] = dv_acc[db][r];
  }
  __syncthreads();
  if (qh == 0) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) dv_acc[db][r] += red[red_idx(db, r)];
  }
  __syncthreads();
  if (qh == 1) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) red[red_idx(db, r)] = dk_acc[db][r];
  }
  __syncthreads();

  // ---- epilogue: dK = scale * dK^T, dV = dV^T (lane = key, regs = d).
  if (qh == 0 && mykey < N) {
    uint16_t* dkr = dK + head + (size_t)mykey * D;
    uint16_t* dvr = dV + head + (size_t)mykey * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 a, b;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a[e] = (dk_acc[db][4 * g + e] + red[red_idx(db, 4 * g + e)]) * scale;
          b[e] = DROP ? dv_acc[db][4 * g + e] * (256.f / (float)(256 - drop.p8))
                      : dv_acc[db][4 * g + e];
        }
        *(bf16x4*)(dkr + 32 * db + 8 * g + 4 * hh) = to_bf16x4(a);
        *(bf16x4*)(dvr + 32 * db + 8 * g + 4 * hh) = to_bf16x4(b);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// dQ kernel: one workgroup per (batch, head, 128-row query block), 4
// wavefronts of 32 query rows, streaming 64-key tiles of K and V through LDS
// (double-buffered) exactly like the forward.  Per tile it recomputes
// S^T = K Q^T and dP^T = V dO^T, forms P^T = exp2(S^T c - lse2) and
// dS^T = P^T (dP^T - D) in-lane (one query per lane), and accumulates
// dQ^T += K^T dS^T with K^T read transposed from LDS.  No atomics: dQ is
// written once, deterministically.
constexpr int kDqBR = 128;
static_assert(FA_SPARSE_BQ % kDqBR == 0, "a dQ block lies in one block-mask row");
constexpr int kDqBC = 64;

// Head dim 128 keeps one wavefront per SIMD (its Q, dO fragments, dQ
// accumulators and the next tile's staging registers do not fit 256 VGPRs
// without spilling); head dim 64 two.
template <int D, bool CAUSAL, bool DROP = false, bool SPARSE = false>
__global__ __launch_bounds__(kThreads, D == 128 ? 1 : 2) void bwd_dq_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
    const float* __restrict__ LSE, const float* __restrict__ Dv,
    uint16_t* __restrict__ dQ, int N, int n_qblk, float c_log2,
    float scale, Dropout drop, const uint8_t* __restrict__ bmask, int H,
    const int32_t* __restrict__ kv_len = nullptr) {
  static_assert(D == 64 || D == 128, "head dimension");
  constexpr int TE = kDqBC * kRS;      // elements per K (or V) tile buffer
  constexpr int CPT = kDqBC * D / 8 / kThreads;   // 16-byte chunks per thread
  __shared__ __attribute__((aligned(16))) uint16_t smem[4 * TE];
  // buffers: K0 | V0 | K1 | V1 (bases opaque: see bwd_dkdv_kernel)
  const int vbase = __builtin_amdgcn_readfirstlane(TE);
  const int buf1 = __builtin_amdgcn_readfirstlane(2 * TE);

  const int BH = gridDim.x / n_qblk;
  int bh, qb;
  block_schedule((int)blockIdx.x, n_qblk, BH, CAUSAL, bh, qb);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = wave_id();
  const int lq = lane & 31;
  const int hh = lane >> 5;
  const int r16 = lane & 15;
  const int dsub = (lane >> 4) & 1;
  const int q0 = qb * kDqBR;
  const int qw0 = q0 + 32 * w;
  const int qw1 = qw0 + 31;
  const int qrow = qw0 + lq;

  const size_t head = (size_t)bh * N * D;
  const uint16_t* Qh = Q + head;
  const uint16_t* Kh = K + head;
  const uint16_t* Vh = V + head;
  const uint16_t* dOh = dO + head;

  // Key padding: keys >= kv_len[b] are masked and not loaded past.
  const int kvlim = kv_len ? min(max(kv_len[bh / H], 0), N) : N;
  int kend = kvlim;
  if (CAUSAL) kend = min(kend, q0 + kDqBR);
  const int ntiles_dense = (kend + kDqBC - 1) / kDqBC;

  // Key tiles to visit: 0 .. ntiles_dense - 1, or (block-sparse: the
  // 128-row block lies in one 256-row block-mask row) the two 64-key tiles
  // of each kept 128-key mask column, the columns listed in LDS; a tile
  // past ntiles_dense is loaded clamped and not computed.
  __shared__ uint16_t col_list[SPARSE ? FA_SPARSE_MAX_KEY_BLOCKS : 1];
  __shared__ int col_count;
  int ntiles = ntiles_dense;
  if constexpr (SPARSE) {
    const int n_mk = (N + FA_SPARSE_BK - 1) / FA_SPARSE_BK;
    const int n_mq = (N + FA_SPARSE_BQ - 1) / FA_SPARSE_BQ;
    const int n_cols = (ntiles_dense + 1) / 2;
    const uint8_t* mrow =
        bmask + ((size_t)(bh % H) * n_mq + q0 / FA_SPARSE_BQ) * n_mk;
    if (w == 0) {
      int cnt = 0;
      for (int base = 0; base < n_cols; base += 64) {
        const int cidx = base + lane;
        const bool keep = cidx < n_cols && mrow[cidx] != 0;
        const unsigned long long bal = __ballot(keep);
        const int below = __builtin_popcountll(bal & ((1ull << lane) - 1ull));
        if (keep) col_list[cnt + below] = (uint16_t)cidx;
        cnt += __builtin_popcountll(bal);
      }
      if (lane == 0) col_count = cnt;
    }
    __syncthreads();
    ntiles = 2 * col_count;
  }
  // Key tile of position t (possibly >= ntiles_dense when sparse).
  auto ktile = [&](int t) -> int {
    if constexpr (SPARSE)
      return 2 * (int)__builtin_amdgcn_readfirstlane((unsigned)col_list[t >> 1]) + (t & 1);
    else
      return t;
  };

  // Q and dO fragments of this lane's query (B operands), LSE and D.
  bf16x8 qf[D / 16], gf[D / 16];
  const int qc = min(qrow, N - 1);
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    const bf16x8 a = *(const bf16x8*)(Qh + (size_t)qc * D + 16 * kk + 8 * hh);
    const bf16x8 g = *(const bf16x8*)(dOh + (size_t)qc * D + 16 * kk + 8 * hh);
    qf[kk] = qrow < N ? a : bf16x8{};
    gf[kk] = qrow < N ? g : bf16x8{};
  }
  float lse2 = INFINITY, dd = 0.f;
  if (qrow < N) {
    const float l = LSE[(size_t)bh * N + qrow];
    lse2 = (l == -INFINITY) ? INFINITY : l * kLog2e;
    dd = Dv[(size_t)bh * N + qrow];
  }

  u32x4 kreg[CPT], vreg[CPT];
  auto load_tile = [&](int j) {
    const int k0 = j * kDqBC;
    const uint16_t* kb = Kh + (size_t)k0 * D;
    const uint16_t* vb = Vh + (size_t)k0 * D;
#pragma unroll
    for (int r = 0; r < CPT; ++r) {
      const int c = tid + kThreads * r;
      const int row = c / (D / 8);
      const int col = 8 * (c % (D / 8));
      const bool ok = k0 + row < N;
      const unsigned off = (unsigned)(min(row, N - 1 - k0) * D + col);
      const u32x4 a = *(const u32x4*)(kb + off);
      const u32x4 b = *(const u32x4*)(vb + off);
      const u32x4 z = u32x4{0, 0, 0, 0};
      kreg[r] = ok ? a : z;
      vreg[r] = ok ? b : z;
    }
  };
  auto store_tile = [&](int buf) {
    uint16_t* kt = smem + (buf ? buf1 : 0);
    uint16_t* vt = kt + vbase;
#pragma unroll
    for (int r = 0; r < CPT; ++r) {
      const int c = tid + kThreads * r;
      const int row = c / (D / 8);
      const int col = 8 * (c % (D / 8));
      *(u32x4*)(&kt[row * kRS + col]) = kreg[r];
      *(u32x4*)(&vt[row * kRS + col]) = vreg[r];
    }
  };

  f32x16 dq_acc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) dq_acc[i] = f32x16{};

  if (ntiles > 0) load_tile(min(ktile(0), ntiles_dense - 1));
  for (int t = 0; t < ntiles; ++t) {
    const int j = ktile(t);
    const int buf = t & 1;
    store_tile(buf);
    __syncthreads();
    if (t + 1 < ntiles) load_tile(min(ktile(t + 1), ntiles_dense - 1));
    if (SPARSE && j >= ntiles_dense) continue;   // second tile past the end
    const int k0 = j * kDqBC;
    if (CAUSAL && k0 > qw1) continue;     // tile wholly in this wave's future
    const uint16_t* kt = smem + (buf ? buf1 : 0);
    const uint16_t* vt = kt + vbase;

    // Per 32-key block kb: S^T = K Q^T and dP^T = V dO^T (keys x queries),
    // then P^T and dS^T in-lane; register r of block kb holds key
    // k0 + 32kb + 8(r/4) + 4hh + r%4 for this lane's query.  One block's
    // S^T and dP^T are live at a time (at head dim 128 two would not fit
    // two wavefronts per SIMD without spilling).
    const bool need_mask = (CAUSAL && k0 + kDqBC - 1 > qw0) || (k0 + kDqBC > kvlim);
    bf16x8 dsb[2][2];
    const float ik = DROP ? 256.f / (float)(256 - drop.p8) : 1.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 s_kb = f32x16{}, dp_kb = f32x16{};
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const int o = (32 * kb + lq) * kRS + 16 * kk + 8 * hh;
        s_kb = mfma32x16(*(const bf16x8*)(&kt[o]), qf[kk], s_kb);
        dp_kb = mfma32x16(*(const bf16x8*)(&vt[o]), gf[kk], dp_kb);
      }
      // Dropout: kz[m] holds the keep bytes of keys k0 + 32kb + 8m + 4hh + b
      // (byte b) for this lane's query; quad lane w makes the generator
      // call of key group w.  dS = P (Z dP / k - D).
      uint32_t kz[4];
      if constexpr (DROP) {
        kz[0] = (uint32_t)((k0 + 32 * kb) / 4 + 2 * (lq & 3) + hh);
        kz[1] = (uint32_t)(qrow >> 2);
        kz[2] = (uint32_t)bh;
        kz[3] = drop.offset;
#pragma unroll
        for (int r = 0; r < 10; ++r) philox_round(kz, drop.k0, drop.k1, r);
        quad_gather(kz);
      }
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        f32x8 x;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int r = 8 * c + e;
          float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s_kb[r], c_log2, -lse2));
          if (need_mask) {
            const int key = k0 + 32 * kb + 8 * (r / 4) + 4 * hh + (r % 4);
            if ((CAUSAL && key > qrow) || key >= kvlim) p = 0.f;
          }
          if constexpr (DROP)
            x[e] = p * ((drop_keep(kz[r / 4], r % 4, drop.p8) ? dp_kb[r] * ik : 0.f) - dd);
          else
            x[e] = p * (dp_kb[r] - dd);
        }
        dsb[kb][c] = to_bf16x8(x);
      }
    }
    // ---- dQ^T += K^T dS^T.  A operand lane (d, hh) element e is
    // K[32kb + 16c + 8(e/4) + 4hh + e%4][d], read transposed.
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int col = 32 * db + 16 * dsub + 4 * (r16 & 3);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const int row = 32 * kb + 16 * c + 4 * hh + (r16 >> 2);
          const i16x4 lo = lds_read_tr16(&kt[row * kRS + col]);
          const i16x4 hi = lds_read_tr16(&kt[(row + 8) * kRS + col]);
          dq_acc[db] = mfma32x16(join_bf16(lo, hi), dsb[kb][c], dq_acc[db]);
        }
      }
    }
  }

  // ---- epilogue: dQ = scale * dQ^T (lane = query, regs = d).
  if (qrow < N) {
    uint16_t* out = dQ + head + (size_t)qrow * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = dq_acc[db][4 * g + e] * scale;
        *(bf16x4*)(out + 32 * db + 8 * g + 4 * hh) = to_bf16x4(x);
      }
    }
  }
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t bwd_rsrc(const uint16_t* p,
                                                           int bytes) {
  // 0x00020000: raw 32-bit data format (untyped loads), range-checked.
  return __builtin_amdgcn_make_buffer_rsrc((void*)p, (short)0, bytes,
                                           0x00020000);
}

// ---------------------------------------------------------------------------
// Pipelined dK/dV kernel: one workgroup per (batch, head, 128-key block), 4
// wavefronts of 32 keys (one per SIMD; at head dim 64 two workgroups share
// a CU, its registers and LDS allowing it).  The K and V fragments of a
// wavefront's keys stay in registers for the whole kernel, so LDS only
// carries the streamed 64-row query tiles (Q, dO, LSE, D).  A tile is two
// 32-row blocks; work item A_c is S = Q_c K^T and dP = dO_c V^T, V_c the
// VALU turning them into P and dS, B_c the products dV^T += dO_c^T P and
// dK^T += Q_c^T dS.  Tile i runs two phases, each 32 MFMAs with one
// block's VALU work interleaved in issue order:
//   phase 1:  A_1(i), B_1(i-1)  ||  V_0(i)
//   phase 2:  B_0(i), A_0(i+1)  ||  V_1(i)
// Tile i is read from iteration i-1 to i+1, so query tiles rotate through
// four LDS stages with one barrier per tile.  Q and dO tiles go from HBM
// straight into LDS by DMA, issued two tiles ahead; LSE and D (64 floats
// each, transformed on the way) pass through wavefront 0's registers.
// Row placement of the streamed tiles of the pipelined backward kernels
// (query tiles in dK/dV, key tiles in dQ).  Two access patterns read a
// tile: row reads (16 lanes on 16 consecutive rows, 16 bytes each) and
// transposed reads (16 or 32 lanes on 4 consecutive rows, 32 or 64 bytes
// each).  Rows are padded to an odd number of 16-byte chunks (272 bytes at
// head dim 128, 144 at 64), and within each group of 16 rows row r sits in
// slot 4 (r mod 4) + r / 4 (its two base-4 digits swapped, so the map is
// its own inverse).  16 consecutive rows then fill 16 distinct slots, and 4
// consecutive rows from a multiple of 4 land in slots 4 apart, so that
// neither pattern meets an LDS bank conflict; a padded stride alone serves
// only one of the two.
__device__ __forceinline__ int tile_slot(int r) {
  return (r & ~15) | ((r & 3) << 2) | ((r >> 2) & 3);
}

constexpr int kKvPBK = 128;

template <bool CAUSAL, bool SPARSE, bool DROP = false, int D = kD>
__global__ __launch_bounds__(256, D == 64 ? 2 : 1) void bwd_dkdv_pipe_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
    const float* __restrict__ LSE, const float* __restrict__ Dv,
    uint16_t* __restrict__ dK, uint16_t* __restrict__ dV,
    const uint8_t* __restrict__ bmask, int H, int N, int n_kblk,
    float c_log2, float scale, Dropout drop,
    const int32_t* __restrict__ kv_len = nullptr) {
  static_assert(D == kD || (D == 64 && !DROP), "head dimension");
  // Query tiles in LDS: rows of D + 8 elements in the slots of tile_slot.
  constexpr int RS = D + 8;
  constexpr int QE = kBQ2 * RS;                  // elements per tile stage
  constexpr int THREADS = 256;
  __shared__ __attribute__((aligned(16))) uint16_t lds_q[4][QE];
  __shared__ __attribute__((aligned(16))) uint16_t lds_g[4][QE];   // dO
  __shared__ __attribute__((aligned(16))) float lds_lse[4][kBQ2];
  __shared__ __attribute__((aligned(16))) float lds_d[4][kBQ2];

  const int BH = gridDim.x / n_kblk;
  // Key blocks with the most visible queries (smallest index) go first.
  const int jb = blockIdx.x / BH;
  const int bh = blockIdx.x % BH;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = wave_id();
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int r16 = lane & 15;
  const int dsub = (lane >> 4) & 1;

  const int kb0 = jb * kKvPBK;
  const int wk0 = kb0 + 32 * w;             // first key of this wavefront
  const int mykey = wk0 + l32;              // this lane's key
  const size_t head = (size_t)bh * N * D;
  const uint16_t* Qh = Q + head;
  const uint16_t* dOh = dO + head;
  const float* LSEh = LSE + (size_t)bh * N;
  const float* Dh = Dv + (size_t)bh * N;

  // K and V fragments of this lane's key (B operands), zero past N.  The
  // sign of the scale is folded into K (exact for bf16), so the exponent
  // scale is positive and masked scores (-inf) give P = 0; a zero scale
  // becomes a tiny positive one.  dK keeps the caller's scale.
  bf16x8 kf[D / 16], vf[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    kf[kk] = mykey < N ? *(const bf16x8*)(K + head + (size_t)mykey * D + 16 * kk + 8 * hh)
                       : bf16x8{};
    vf[kk] = mykey < N ? *(const bf16x8*)(V + head + (size_t)mykey * D + 16 * kk + 8 * hh)
                       : bf16x8{};
  }
  if (c_log2 < 0.f) {
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) kf[kk] = -kf[kk];
    c_log2 = -c_log2;
  }
  c_log2 = fmaxf(c_log2, 1e-30f);

  const int n_qt = (N + kBQ2 - 1) / kBQ2;
  // Key padding: keys >= kv_len[b] are masked (a block wholly past it
  // visits no query tile and writes dK = dV = 0).
  const int kvlim = kv_len ? min(max(kv_len[bh / H], 0), N) : N;
  const int it0 = CAUSAL ? kb0 / kBQ2 : 0;

  // ---- query tiles to visit.  Dense: it0 .. n_qt - 1.  Block-sparse: the
  // workgroup's 128 keys are one block-mask column; the 64-row query tiles
  // whose block row keeps it are compacted into an LDS list.
  __shared__ uint16_t qt_list[SPARSE ? kSparseMaxTiles : 1];
  __shared__ int qt_count;
  int n_vis = n_qt - it0;
  if constexpr (SPARSE) {
    const int n_mk = (N + FA_SPARSE_BK - 1) / FA_SPARSE_BK;
    const int n_mq = (N + FA_SPARSE_BQ - 1) / FA_SPARSE_BQ;
    const uint8_t* mcol = bmask + (size_t)(bh % H) * n_mq * n_mk + jb;
    if (w == 0) {
      int cnt = 0;
      for (int base = it0; base < n_qt; base += 64) {
        const int q = base + lane;
        const bool keep =
            q < n_qt && mcol[(size_t)(q * kBQ2 / FA_SPARSE_BQ) * n_mk] != 0;
        const unsigned long long bal = __ballot(keep);
        const int below = __builtin_popcountll(bal & ((1ull << lane) - 1ull));
        if (keep) qt_list[cnt + below] = (uint16_t)q;
        cnt += __builtin_popcountll(bal);
      }
      if (lane == 0) qt_count = cnt;
    }
    __syncthreads();
    n_vis = qt_count;
  }
  if (kb0 >= kvlim) n_vis = 0;
  // Query tile of visit i (clamped; it0 + i when dense).
  auto qtile = [&](int i) -> int {
    if constexpr (SPARSE)
      return (int)__builtin_amdgcn_readfirstlane((unsigned)qt_list[max(min(i, n_vis - 1), 0)]);
    else
      return it0 + i;
  };

  // The K and V fragments have arrived before any DMA is issued (a wait
  // the compiler can see, so that it places none of its own inside the
  // tile loop).
  __builtin_amdgcn_s_waitcnt(kWaitVm0);

  // ---- query-tile staging.  Q and dO: DMA instruction u of wavefront w
  // fills the 1 KB of the (padded) stage at 1024 (w + 4u), 16 bytes per
  // lane; lanes on row padding, and rows past N, read zeros.
  constexpr int RCH = RS / 8;                       // 16-B slots per row
  constexpr int TI = kBQ2 * RCH / 64;                // DMA instructions per tile
  constexpr int TIW = (TI + 3) / 4;
  static_assert(QE % 512 == 0, "tile stage must be whole 1 KB blocks");
  unsigned toff[TIW];
#pragma unroll
  for (int u = 0; u < TIW; ++u) {
    // slot p / RCH holds row tile_slot(p / RCH) (the map is an involution)
    const int p = 64 * (w + 4 * u) + lane, row = tile_slot(p / RCH), c = p % RCH;
    toff[u] = c < D / 8 ? (unsigned)((row * D + 8 * c) * 2) : (1u << 30);
  }
  const unsigned lds_q0 = lds_addr(&lds_q[0][0]);
  const unsigned lds_g0 = lds_addr(&lds_g[0][0]);
  float lse_r = 0.f, d_r = 0.f;
  int stats_q = 0;
  auto dma_tile = [&](int it, int st) {
    const int qt0 = it * kBQ2;
    const int bytes = min(N - qt0, kBQ2) * D * 2;
    const auto rq = bwd_rsrc(Qh + (size_t)qt0 * D, bytes);
    const auto rg = bwd_rsrc(dOh + (size_t)qt0 * D, bytes);
    const unsigned off = (unsigned)(st * QE * 2);
#pragma unroll
    for (int u = 0; u < TIW; ++u)
      if (TI % 4 == 0 || w + 4 * u < TI) {
        lds_dma16(rq, lds_q0 + off + 1024u * (w + 4 * u), toff[u]);
        lds_dma16(rg, lds_g0 + off + 1024u * (w + 4 * u), toff[u]);
      }
  };
  // LSE and D of a tile: loaded raw one iteration ahead, turned into the
  // per-row exponent offset at the store (so no wait falls mid-tile).
  auto load_stats = [&](int it) {
    if (w == 0) {
      stats_q = it * kBQ2 + lane;
      const int q = max(min(stats_q, N - 1), 0);
      lse_r = LSEh[q];
      d_r = Dh[q];
    }
  };
  // With dropout the dP accumulators start at -D times the keep
  // probability (see the phase).
  const float kp = DROP ? (float)(256 - drop.p8) * (1.f / 256.f) : 1.f;
  auto store_stats = [&](int st) {
    if (w == 0) {
      // Rows past N (and rows without any visible key) get +inf, so that
      // exp2(s - lse) = 0 for every key.
      const bool in = stats_q < N;
      const float l = in ? lse_r : INFINITY;
      lds_lse[st][lane] = (l == -INFINITY) ? INFINITY : l * kLog2e;
      lds_d[st][lane] = in ? -d_r * kp : 0.f;   // -D: the dP accumulators start there
    }
  };

  f32x16 dk_acc[D / 32], dv_acc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) {
    dk_acc[i] = f32x16{};
    dv_acc[i] = f32x16{};
  }
  f32x16 s[2], dp[2];          // S, dP of each block (lane = key)
  bf16x8 pb[2][2], dsb[2][2];  // P, dS of each block in bf16, 16-row halves

  // ---- dropout bytes.  kz[m]: keep bytes of the VALU block's rows
  // 8m + 4hh + a (byte a) for this lane's key, i.e. register 4m + a.  Quad
  // lane w (keys 4kb .. 4kb+3) makes the generator call of row group w,
  // transposes its bytes so that word b holds key 4kb + b, and the quad
  // exchange hands each lane its key's word of every call.  A phase
  // computes the bytes of the next phase's VALU block (kzn) in the MFMA
  // slots after its own VALU work, and takes them over at its start.
  uint32_t kz[4], kzn[4];
  auto gen_begin = [&](int qt, int c) __attribute__((always_inline)) {
    kzn[0] = (uint32_t)(mykey >> 2);
    kzn[1] = (uint32_t)(qt * (kBQ2 / 4) + 8 * c + 2 * (l32 & 3) + hh);
    kzn[2] = (uint32_t)bh;
    kzn[3] = drop.offset;
  };
  auto gen_end = [&]() __attribute__((always_inline)) {
    byte_transpose(kzn);
    quad_gather(kzn);
  };

  // ---- one phase.  A: S, dP of block ca from stage sta.  B: dV, dK of
  // block cb from stage stb.  VALU: P, dS of block cv with LSE / D from
  // stage stv.  B_FIRST orders the B products before the A ones.  The
  // operand of MFMA slot m is read from LDS kPf slots ahead, and the ring
  // runs on across phases: the last kPf slots of a phase read the first
  // operands of the next phase (stages nsta, nstb, blocks nca, ncb; its
  // B_FIRST is the opposite), and the LSE / -D rows of the next phase are
  // read kPf slots before its start, so no phase begins by waiting for LDS.
  constexpr int kA = 2 * (D / 16);       // S and dP MFMAs
  constexpr int kB = 4 * (D / 32);       // dV and dK MFMAs
  constexpr int kN = kA + kB;
  constexpr int kPf = 4;
  static_assert(kN % kPf == 0, "the ring position repeats per phase");
  // VALU elements per MFMA slot: the 16 elements of a block run through a
  // three-slot pipeline, so a phase of kN slots carries one per slot at
  // head dim 128 (32 slots) and two at head dim 64 (16 slots).
  constexpr int kG = kN >= 18 ? 1 : 2;
  static_assert(kG * (kN - 2) >= 16, "the VALU pipeline fits the phase");
  auto fetch = [&](auto b_first, int i, int sta, int ca, int stb,
                   int cb) __attribute__((always_inline)) -> bf16x8 {
    constexpr bool BF = decltype(b_first)::value;
    const bool is_a = BF ? (i >= kB) : (i < kA);
    if (is_a) {
      const int ai = BF ? i - kB : i;
      const int kk = ai / 2;
      const uint16_t* t = (ai % 2 == 0) ? lds_q[sta] : lds_g[sta];
      return *(const bf16x8*)(&t[(32 * ca + tile_slot(l32)) * RS + 16 * kk + 8 * hh]);
    }
    const int bi = BF ? i : i - kA;
    const int which = bi / (kB / 2);           // 0: dO^T (dV), 1: Q^T (dK)
    const int h = (bi % (kB / 2)) / (D / 32), db = bi % (D / 32);
    const uint16_t* t = which == 0 ? lds_g[stb] : lds_q[stb];
    const int col = 32 * db + 16 * dsub + 4 * (r16 & 3);
    const int row = 32 * cb + 16 * h + 4 * hh + (r16 >> 2);
    return join_bf16(lds_read_tr16(&t[tile_slot(row) * RS + col]),
                     lds_read_tr16(&t[tile_slot(row + 8) * RS + col]));
  };
  // LSE of the lane's 16 rows of block cv, -D of those of block ca (and,
  // with dropout, of block cv): register r <-> row 32 c + 8 (r / 4) + 4 hh
  // + r % 4.  dP accumulates onto -D, so the VALU forms dS = P (dP - D)
  // with one product.
  bf16x8 op[kPf];
  f32x4 l4[4], nd4[4], nv4[4];
  auto fetch_rows = [&](int sta, int ca, int stv, int cv) __attribute__((always_inline)) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      l4[g] = *(const f32x4*)(&lds_lse[stv][32 * cv + 8 * g + 4 * hh]);
      nd4[g] = *(const f32x4*)(&lds_d[sta][32 * ca + 8 * g + 4 * hh]);
      if constexpr (DROP)
        nv4[g] = *(const f32x4*)(&lds_d[stv][32 * cv + 8 * g + 4 * hh]);
    }
  };
  // Operands and rows of the first phase (the ring's start).
  auto prefetch = [&](auto b_first, int sta, int ca, int stb, int cb, int stv,
                      int cv) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kPf; ++i) op[i] = fetch(b_first, i, sta, ca, stb, cb);
    fetch_rows(sta, ca, stv, cv);
  };
  auto phase = [&](auto b_first, int sta, int ca, int stb, int cb,
                   int stv, int cv, int qtn, int cvn, int nsta, int nca,
                   int nstb, int ncb, int nstv, int ncv) {
    constexpr bool BF = decltype(b_first)::value;
    using NextBF = std::integral_constant<bool, !BF>;
    f32x4 lv[4];
    f32x16 negd, negd_v;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      lv[g] = l4[g];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        negd[4 * g + e] = nd4[g][e];
        if constexpr (DROP) negd_v[4 * g + e] = nv4[g][e];
      }
    }
    // Dropout: with Z the keep mask and k the keep probability,
    // dS = P (Z dP'/k - D) = (P/k) (Z ? dP' - k D : -k D), where dP' =
    // dO V^T and the accumulator holds dP' - k D; dV takes P Z.  The 1/k
    // of both is applied at the end.
    if constexpr (DROP) {
#pragma unroll
      for (int m = 0; m < 4; ++m) kz[m] = kzn[m];
      gen_begin(qtn, cvn);
    }
    // VALU: 16 elements as a three-stage pipeline over the MFMA slots
    // (FMA, then exp2, then dS and, per 8 elements, the bf16 conversions).
    float x[16], pe[16], dsv[16];
#pragma unroll
    for (int m = 0; m < kN; ++m) {
      const bf16x8 a = op[m % kPf];
      if (m + kPf < kN)
        op[m % kPf] = fetch(b_first, m + kPf, sta, ca, stb, cb);
      else
        op[m % kPf] = fetch(NextBF{}, m + kPf - kN, nsta, nca, nstb, ncb);
      if (m == kN - kPf) fetch_rows(nsta, nca, nstv, ncv);
      const bool is_a = BF ? (m >= kB) : (m < kA);
      if (is_a) {
        const int ai = BF ? m - kB : m;
        const int kk = ai / 2;
        if (ai % 2 == 0)
          s[ca] = mfma32x16(a, kf[kk], kk == 0 ? f32x16{} : s[ca]);
        else
          dp[ca] = mfma32x16(a, vf[kk], kk == 0 ? negd : dp[ca]);
      } else {
        const int bi = BF ? m : m - kA;
        const int which = bi / (kB / 2);
        const int h = (bi % (kB / 2)) / (D / 32), db = bi % (D / 32);
        if (which == 0)
          mfma_agpr(dv_acc[db], a, pb[cb][h]);
        else
          mfma_agpr(dk_acc[db], a, dsb[cb][h]);
      }
#pragma unroll
      for (int u = 0; u < kG; ++u) {
      const int mf = kG * m + u, me = kG * (m - 1) + u, md = kG * (m - 2) + u;
      if (mf < 16) x[mf] = __builtin_fmaf(s[cv][mf], c_log2, -lv[mf / 4][mf % 4]);
      if (m >= 1 && me < 16) pe[me] = __builtin_amdgcn_exp2f(x[me]);
      if (m >= 2 && md < 16) {
        const int el = md;
        if constexpr (DROP) {
          const bool kept = drop_keep(kz[el / 4], el % 4, drop.p8);
          dsv[el] = pe[el] * (kept ? dp[cv][el] : negd_v[el]);
          if (!kept) pe[el] = 0.f;
        } else {
          dsv[el] = pe[el] * dp[cv][el];
        }
        if (el % 8 == 7) {
          f32x8 vp, vd;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            vp[e] = pe[el - 7 + e];
            vd[e] = dsv[el - 7 + e];
          }
          pb[cv][el / 8] = to_bf16x8(vp);
          dsb[cv][el / 8] = to_bf16x8(vd);
        }
      }
      }
      if constexpr (DROP) {
        static_assert(kN >= 29, "generator rounds fit after the VALU work");
        if (m >= 18 && m < 28) philox_round(kzn, drop.k0, drop.k1, m - 18);
        if (m == 28) gen_end();
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // Keep the VALU work in this phase: without a use here the compiler
    // sinks it past the masking branch that follows.
    asm volatile("" : "+v"(pb[cv][0]), "+v"(pb[cv][1]), "+v"(dsb[cv][0]),
                 "+v"(dsb[cv][1]));
  };

  // ---- mask block c of query tile qt where needed (causal diagonal, keys
  // past N; rows past N already have P = 0 through LSE = +inf).
  auto mask_block = [&](int c, int qt) {
    const int qb0 = qt * kBQ2 + 32 * c;
    const bool need_mask = (CAUSAL && wk0 + 31 > qb0) || (wk0 + 32 > kvlim);
    if (need_mask) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int q = qb0 + 8 * (r / 4) + 4 * hh + (r % 4);
        if ((CAUSAL && mykey > q) || mykey >= kvlim) s[c][r] = -INFINITY;
      }
    }
  };

  // ---- dV, dK of block 1 of the last tile (no VALU work left).
  auto b_only = [&](int stb) {
#pragma unroll
    for (int bi = 0; bi < 4 * (D / 32); ++bi) {
      const int which = bi / (2 * (D / 32));
      const int h = (bi % (2 * (D / 32))) / (D / 32), db = bi % (D / 32);
      const uint16_t* t = which == 0 ? lds_g[stb] : lds_q[stb];
      const int col = 32 * db + 16 * dsub + 4 * (r16 & 3);
      const int row = 32 + 16 * h + 4 * hh + (r16 >> 2);
      const bf16x8 a = join_bf16(lds_read_tr16(&t[tile_slot(row) * RS + col]),
                                 lds_read_tr16(&t[tile_slot(row + 8) * RS + col]));
      if (which == 0)
        mfma_agpr(dv_acc[db], a, pb[1][h]);
      else
        mfma_agpr(dk_acc[db], a, dsb[1][h]);
    }
  };

  int free_stage = 2;   // a stage no wavefront reads after the tile loop
  if (n_vis > 0) {
    const int last = n_vis - 1;      // list positions
    // Prologue: the first tile in stage 0, the second in stage 1 (its LSE /
    // D in registers); zeros in stage 3 (the tile before the first, whose
    // block 1 the first phase multiplies by P = dS = 0); A_0 of the first.
    const int e0 = qtile(0);
    dma_tile(e0, 0);
    if (last >= 1) dma_tile(qtile(1), 1);
    load_stats(e0);
    store_stats(0);
    load_stats(qtile(min(1, last)));
    for (int e = tid; e < QE / 8; e += THREADS) {
      *(u32x4*)(&lds_q[3][8 * e]) = u32x4{0, 0, 0, 0};
      *(u32x4*)(&lds_g[3][8 * e]) = u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        pb[c][h] = bf16x8{};
        dsb[c][h] = bf16x8{};
      }
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
    f32x16 negd0;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 nd = *(const f32x4*)(&lds_d[0][8 * g + 4 * hh]);
#pragma unroll
      for (int e = 0; e < 4; ++e) negd0[4 * g + e] = nd[e];
    }
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      const int o = tile_slot(l32) * RS + 16 * kk + 8 * hh;
      s[0] = mfma32x16(*(const bf16x8*)(&lds_q[0][o]), kf[kk], kk == 0 ? f32x16{} : s[0]);
      dp[0] = mfma32x16(*(const bf16x8*)(&lds_g[0][o]), vf[kk], kk == 0 ? negd0 : dp[0]);
    }
    mask_block(0, e0);
    if constexpr (DROP) {
      gen_begin(e0, 0);
#pragma unroll
      for (int r = 0; r < 10; ++r) philox_round(kzn, drop.k0, drop.k1, r);
      gen_end();
    }
    agpr_hazard_pad();   // zero-filled accumulators -> first MFMA

    // Visited tile i (list position) in stage i % 4.  Iteration i publishes
    // tile i+1 (its DMA has landed, its LSE / D are stored), then issues
    // tile i+2 into the stage of tile i-2, last read in iteration i-1.
    int sp = 3, s0 = 0, s1 = 1;   // stages of tiles i-1, i, i+1
    prefetch(std::false_type{}, s0, 1, sp, 1, s0, 0);
    for (int i = 0; i < n_vis; ++i) {
      const int ei = qtile(i), ei1 = qtile(i + 1), ei2 = qtile(min(i + 2, last));
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      store_stats(s1);
      __syncthreads();
      if (i + 2 <= last) dma_tile(ei2, (s1 + 1) & 3);
      load_stats(ei2);
      // phase 1: A_1(i), B_1(i-1) || V_0(i); the ring then reads phase 2's
      phase(std::false_type{}, s0, 1, sp, 1, s0, 0, ei, 1, s1, 0, s0, 0, s0, 1);
      mask_block(1, ei);
      // phase 2: B_0(i), A_0(i+1) || V_1(i); the ring then reads phase 1 of
      // tile i+1 (stages s1 and s0 after the rotation below)
      phase(std::true_type{}, s1, 0, s0, 0, s0, 1, ei1, 0, s1, 1, s0, 1, s1, 0);
      if (i + 1 < n_vis) mask_block(0, ei1);
      sp = s0;
      s0 = s1;
      s1 = (s1 + 1) & 3;
    }
    b_only(sp);
    agpr_hazard_pad();   // last MFMA -> epilogue reads
    // Tile last+2's stage: no transfer fills it and no wavefront reads it
    // after the last iteration's barrier.
    free_stage = s1;
  }

  // ---- epilogue: dK = scale * dK^T, dV = dV^T (lane = key, regs = d);
  // with dropout both are divided by the keep probability.  A lane holds
  // 8-byte pieces of its key's row, so stores straight from the registers
  // would touch 32 rows per instruction; instead each wavefront writes its
  // 32 rows in bf16 to its own area of the free stage (rows padded to
  // D + 8 elements) and reads them back 16 bytes per lane, so that every
  // store instruction writes whole rows.
  const float sk = DROP ? scale / kp : scale, sv = DROP ? 1.f / kp : 1.f;
  constexpr int ES = D + 8;                  // row stride of the area
  constexpr int CPR = D / 8;                 // 16-byte pieces per row
  static_assert(2 * 32 * ES <= QE, "two wavefronts' rows fit a stage array");
  uint16_t* area = (w < 2 ? lds_q[free_stage] : lds_g[free_stage]) + (w & 1) * 32 * ES;
  auto store_rows = [&](f32x16* acc, float mul, uint16_t* out) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 a;
#pragma unroll
        for (int e = 0; e < 4; ++e) a[e] = acc[db][4 * g + e] * mul;
        *(bf16x4*)(area + l32 * ES + 32 * db + 8 * g + 4 * hh) = to_bf16x4(a);
      }
    }
#pragma unroll
    for (int i = 0; i < 32 * CPR / 64; ++i) {
      const int row = i * (64 / CPR) + lane / CPR, c = lane % CPR;
      const u32x4 v = *(const u32x4*)(area + row * ES + 8 * c);
      if (wk0 + row < N) *(u32x4*)(out + head + (size_t)(wk0 + row) * D + 8 * c) = v;
    }
  };
  store_rows(dk_acc, sk, dK);
  store_rows(dv_acc, sv, dV);
}

// ---------------------------------------------------------------------------
// Pipelined dQ kernel: one workgroup per (batch, head, 256-row query block),
// 8 wavefronts of 32 query rows (two per SIMD).  The key axis is walked in
// half-tiles of 32 keys, t = 2j + kb; step t issues
//   S^T_{t+1} = K Q^T and dP^T_{t+1} = V dO^T on the matrix cores while the
//   VALU forms P_t = exp2(c S^T_t - lse) and dS^T_t = P_t (dP^T_t - D),
//   then dQ^T += K_t^T dS^T_t,
// with MFMAs and VALU work interleaved one by one in issue order.  K and V
// tile j are read in tiles j-1 and j; they go from HBM straight into LDS by
// DMA, issued three tiles ahead into four stages (one barrier per tile).
// The DMA descriptor ends at the head's last key: keys past N read as zero.
constexpr int kDqPBR = 256;

template <bool CAUSAL, bool SPARSE, bool DROP = false, int D = kD>
__global__ __launch_bounds__(512, 2) void bwd_dq_pipe_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
    const float* __restrict__ LSE, const float* __restrict__ Dv,
    uint16_t* __restrict__ dQ, const uint8_t* __restrict__ bmask, int H,
    int N, int n_qblk, float c_log2, float scale, Dropout drop,
    const int32_t* __restrict__ kv_len = nullptr) {
  static_assert(!SPARSE || kDqPBR == FA_SPARSE_BQ, "a workgroup is a mask row");
  static_assert(D == kD || (D == 64 && !DROP), "head dimension");
  // K/V tiles in LDS: rows of D + 8 elements in the slots of tile_slot.
  constexpr int RS = D + 8;
  constexpr int TE = kDqBC * RS;                  // elements per tile stage
  constexpr int THREADS = 512;
  constexpr int NW = THREADS / 64;
  __shared__ __attribute__((aligned(16))) uint16_t lds_k[4][TE];
  __shared__ __attribute__((aligned(16))) uint16_t lds_v[4][TE];

  const int BH = gridDim.x / n_qblk;
  int bh, qb;
  block_schedule((int)blockIdx.x, n_qblk, BH, CAUSAL, bh, qb);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = wave_id();
  const int lq = lane & 31;
  const int hh = lane >> 5;
  const int r16 = lane & 15;
  const int dsub = (lane >> 4) & 1;
  const int q0 = qb * kDqPBR;
  const int qlo = q0 + 32 * w;
  const int qrow = qlo + lq;

  // Key padding: keys >= kv_len[b] are masked and not loaded past.
  const int kvlim = kv_len ? min(max(kv_len[bh / H], 0), N) : N;
  int kend = kvlim;
  if (CAUSAL) kend = min(kend, q0 + kDqPBR);
  int ntiles = (kend + kDqBC - 1) / kDqBC;
  int kend_w = kvlim;
  if (CAUSAL) kend_w = min(kend_w, qlo + 32);
  int nt_w = (kend_w + kDqBC - 1) / kDqBC;

  // ---- block-sparse: the key tiles this workgroup's block-mask row keeps,
  // in order, as a list in LDS; ntiles and nt_w then count list entries.
  __shared__ uint16_t tile_list[SPARSE ? kSparseMaxTiles : 1];
  __shared__ int tile_count;
  if constexpr (SPARSE) {
    const int n_mk = (N + FA_SPARSE_BK - 1) / FA_SPARSE_BK;
    const int n_mq = (N + kDqPBR - 1) / kDqPBR;
    const uint8_t* mrow = bmask + ((size_t)(bh % H) * n_mq + qb) * n_mk;
    if (w == 0) {
      int cnt = 0;
      for (int base = 0; base < ntiles; base += 64) {
        const int j = base + lane;      // key tile j lies in mask column j/2
        const bool keep = j < ntiles && mrow[j >> 1] != 0;
        const unsigned long long bal = __ballot(keep);
        const int below = __builtin_popcountll(bal & ((1ull << lane) - 1ull));
        if (keep) tile_list[cnt + below] = (uint16_t)j;
        cnt += __builtin_popcountll(bal);
      }
      if (lane == 0) tile_count = cnt;
    }
    __syncthreads();
    const int dense_nt_w = nt_w;
    ntiles = tile_count;
    nt_w = ntiles;
    if (CAUSAL) {
      nt_w = 0;
      for (int base = 0; base < ntiles; base += 64) {
        const int t = base + lane;
        nt_w += __builtin_popcountll(
            __ballot(t < ntiles && (int)tile_list[t] < dense_nt_w));
      }
    }
  }
  // Key tile of list position t (clamped; the position itself when dense).
  auto ktile = [&](int t) -> int {
    if constexpr (SPARSE)
      return (int)__builtin_amdgcn_readfirstlane((unsigned)tile_list[max(min(t, ntiles - 1), 0)]);
    else
      return t;
  };

  const size_t head = (size_t)bh * N * D;
  const uint16_t* Qh = Q + head;
  const uint16_t* Kh = K + head;
  const uint16_t* Vh = V + head;
  const uint16_t* dOh = dO + head;

  // Q and dO fragments of this lane's query (B operands), LSE and D.
  bf16x8 qf[D / 16], gf[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    qf[kk] = qrow < N ? *(const bf16x8*)(Qh + (size_t)qrow * D + 16 * kk + 8 * hh)
                      : bf16x8{};
    gf[kk] = qrow < N ? *(const bf16x8*)(dOh + (size_t)qrow * D + 16 * kk + 8 * hh)
                      : bf16x8{};
  }
  // The sign of the scale is folded into Q (bf16 negation is exact), so the
  // exponent scale is positive and masked scores (-inf) give P = 0; a zero
  // scale becomes a tiny positive one.  dQ keeps the caller's scale.
  if (c_log2 < 0.f) {
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) qf[kk] = -qf[kk];
    c_log2 = -c_log2;
  }
  c_log2 = fmaxf(c_log2, 1e-30f);
  float lse2 = INFINITY, dd = 0.f;   // rows past N (and empty rows): P = 0
  if (qrow < N) {
    const float l = LSE[(size_t)bh * N + qrow];
    lse2 = (l == -INFINITY) ? INFINITY : l * kLog2e;
    dd = Dv[(size_t)bh * N + qrow];
  }
  // dP^T accumulates onto -D (one query per lane), so the VALU forms
  // dS = P (dP - D) with one product.  Dropout (Z the keep mask, k the
  // keep probability): dS = P (Z dP'/k - D) = (P/k) (Z ? dP' - k D : -k D)
  // with dP' = dO V^T; the accumulator starts at -k D and the 1/k is
  // applied at the end.
  const float kp = DROP ? (float)(256 - drop.p8) * (1.f / 256.f) : 1.f;
  const float negd_s = -dd * kp;
  f32x16 negd;
#pragma unroll
  for (int r = 0; r < 16; ++r) negd[r] = negd_s;

  // Every register operand has arrived before any DMA is issued (a wait
  // the compiler can see, so that it places none of its own inside the
  // tile loop).
  __builtin_amdgcn_s_waitcnt(kWaitVm0);

  // ---- K/V tile DMA: instruction u of wavefront w fills the 1 KB of the
  // (padded) stage at 1024 (w + NW u), 16 bytes per lane; lanes on row
  // padding, and keys past N, read zeros.
  constexpr int RCH = RS / 8;                       // 16-B slots per row
  constexpr int TI = kDqBC * RCH / 64;               // DMA instructions per tile
  constexpr int TIW = (TI + NW - 1) / NW;
  constexpr int kMinBatch = 2 * (TI / NW);           // fewest a wave issues per tile
  static_assert(TE % 512 == 0 && kMinBatch < 16, "DMA tile layout");
  unsigned toff[TIW];
#pragma unroll
  for (int u = 0; u < TIW; ++u) {
    // slot p / RCH holds row tile_slot(p / RCH) (the map is an involution)
    const int p = 64 * (w + NW * u) + lane, row = tile_slot(p / RCH), c = p % RCH;
    toff[u] = c < D / 8 ? (unsigned)((row * D + 8 * c) * 2) : (1u << 30);
  }
  const unsigned lds_k0 = lds_addr(&lds_k[0][0]);
  const unsigned lds_v0 = lds_addr(&lds_v[0][0]);
  auto dma_kv = [&](int j, int st) {
    const int k0 = j * kDqBC;
    const int bytes = min(N - k0, kDqBC) * D * 2;
    const auto rk = bwd_rsrc(Kh + (size_t)k0 * D, bytes);
    const auto rv = bwd_rsrc(Vh + (size_t)k0 * D, bytes);
    const unsigned off = (unsigned)(st * TE * 2);
#pragma unroll
    for (int u = 0; u < TIW; ++u)
      if (TI % NW == 0 || w + NW * u < TI) {
        lds_dma16(rk, lds_k0 + off + 1024u * (w + NW * u), toff[u]);
        lds_dma16(rv, lds_v0 + off + 1024u * (w + NW * u), toff[u]);
      }
  };

  f32x16 dq_acc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) dq_acc[i] = f32x16{};
  f32x16 s[2], dp[2];        // S^T, dP^T of a half-tile, by parity
  bf16x8 dsb[2];             // dS^T in bf16, 16-key halves

  // ---- dropout bytes.  kz[m]: keep bytes of the VALU half-tile, key group
  // m (keys k0 + 8m + 4hh + b, byte b) for this lane's query, i.e.
  // register 4m + b.  Quad lane w makes the generator call of key group w
  // for the quad's four queries; a step computes the bytes of the next
  // step's half-tile in its last MFMA slots, after its own VALU work (one
  // set of registers: the kernel has none to spare).
  uint32_t kz[4];
  auto gen_begin = [&](int k0) __attribute__((always_inline)) {
    kz[0] = (uint32_t)(k0 / 4 + 2 * (lq & 3) + hh);
    kz[1] = (uint32_t)(qrow >> 2);
    kz[2] = (uint32_t)bh;
    kz[3] = drop.offset;
  };

  // ---- one step.  XS: parity receiving S^T, dP^T of the next half-tile
  // (stage stn, 32-key half kbn); the VALU and dQ take the current one
  // (parity 1 - XS, K stage stc, half kbc).
  auto step = [&](auto xs_tag, int stn, int kbn, int stc, int kbc, int k0n) {
    constexpr int XS = decltype(xs_tag)::value;
    constexpr int XE = 1 - XS;
    constexpr int kS = D / 16;           // MFMAs for S^T (and for dP^T)
    constexpr int kQ = 2 * (D / 32);     // MFMAs for dQ^T
    constexpr int kN = 2 * kS + kQ;
    constexpr int kPf = 3;
    // VALU elements per MFMA slot (the 16 elements' three-slot pipeline
    // over a step of kN slots): one at head dim 128, two at head dim 64.
    constexpr int kG = kN >= 18 ? 1 : 2;
    static_assert(kG * (kN - 2) >= 16, "the VALU pipeline fits the step");
    auto fetch = [&](int i) -> bf16x8 {
      if (i < kS)
        return *(const bf16x8*)(&lds_k[stn][(32 * kbn + tile_slot(lq)) * RS + 8 * hh + 16 * i]);
      if (i < 2 * kS)
        return *(const bf16x8*)(&lds_v[stn][(32 * kbn + tile_slot(lq)) * RS + 8 * hh + 16 * (i - kS)]);
      const int pi = i - 2 * kS;
      const int h = pi / (D / 32), db = pi % (D / 32);
      const int col = 32 * db + 16 * dsub + 4 * (r16 & 3);
      const int row = 32 * kbc + 16 * h + 4 * hh + (r16 >> 2);
      return join_bf16(lds_read_tr16(&lds_k[stc][tile_slot(row) * RS + col]),
                       lds_read_tr16(&lds_k[stc][tile_slot(row + 8) * RS + col]));
    };
    // Operand of slot m: the S^T and dP^T products alternate (S_0, dP_0,
    // S_1, dP_1, ...) so that no MFMA is issued right after one that
    // accumulates into the same registers (a dependent issue waits out the
    // instruction's latency); the dQ products follow.
    auto op_of = [](int m) constexpr -> int {
      return m < 2 * kS ? ((m & 1) ? kS + (m >> 1) : (m >> 1)) : m;
    };
    bf16x8 op[kPf];
#pragma unroll
    for (int i = 0; i < kPf; ++i) op[i] = fetch(op_of(i));
    // VALU: 16 elements as a three-stage pipeline over the MFMA slots
    // (FMA, then exp2, then dS and, per 8 elements, the bf16 conversion);
    // the dQ MFMAs come last, after each half of dS^T is converted.
    float x[16], pe[16], dsv[16];
#pragma unroll
    for (int m = 0; m < kN; ++m) {
      const bf16x8 a = op[m % kPf];
      if (m + kPf < kN) op[m % kPf] = fetch(op_of(m + kPf));
      const int i = op_of(m);
      if (i < kS) {
        s[XS] = mfma32x16(a, qf[i], i == 0 ? f32x16{} : s[XS]);
      } else if (i < 2 * kS) {
        const int kk = i - kS;
        if constexpr (DROP) {
          // The splat of -k D is rebuilt per step from one register (the
          // dropout variant has no registers to keep all sixteen live).
          if (kk == 0) {
            float nd = negd_s;
            asm volatile("" : "+v"(nd));
            f32x16 c0;
#pragma unroll
            for (int r = 0; r < 16; ++r) c0[r] = nd;
            dp[XS] = mfma32x16(a, gf[kk], c0);
          } else {
            dp[XS] = mfma32x16(a, gf[kk], dp[XS]);
          }
        } else {
          dp[XS] = mfma32x16(a, gf[kk], kk == 0 ? negd : dp[XS]);
        }
      } else {
        // Half 0 of dS^T (converted in slot 9) feeds the first D/32 of
        // these MFMAs, half 1 (converted in slot 17) the last D/32, which
        // start at slot 2 kS + D/32 = 20: each half is ready before use.
        const int pi = i - 2 * kS;
        dq_acc[pi % (D / 32)] = mfma32x16(a, dsb[pi / (D / 32)], dq_acc[pi % (D / 32)]);
      }
#pragma unroll
      for (int u = 0; u < kG; ++u) {
      const int mf = kG * m + u, me = kG * (m - 1) + u, md = kG * (m - 2) + u;
      if (mf < 16) x[mf] = __builtin_fmaf(s[XE][mf], c_log2, -lse2);
      if (m >= 1 && me < 16) pe[me] = __builtin_amdgcn_exp2f(x[me]);
      if (m >= 2 && md < 16) {
        const int el = md;
        if constexpr (DROP)
          dsv[el] = pe[el] * (drop_keep(kz[el / 4], el % 4, drop.p8) ? dp[XE][el]
                                                                    : negd_s);
        else
          dsv[el] = pe[el] * dp[XE][el];
        if (el % 8 == 7) {
          f32x8 v;
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = dsv[el - 7 + e];
          dsb[el / 8] = to_bf16x8(v);
        }
      }
      }
      if constexpr (DROP) {
        // Slots 18 .. 22: two generator rounds each; slot 23: exchange.
        static_assert(kN == 24, "generator slots");
        if (m == 18) gen_begin(k0n);
        if (m >= 18 && m < 23) {
          philox_round(kz, drop.k0, drop.k1, 2 * (m - 18));
          philox_round(kz, drop.k0, drop.k1, 2 * (m - 18) + 1);
        }
        if (m == 23) quad_gather(kz);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- mask the half-tile (j, kb) held in parity x where needed.
  auto mask_half = [&](int x, int j, int kb) {
    const int k0 = j * kDqBC + 32 * kb;
    const bool need_mask = (CAUSAL && k0 + 31 > qlo) || (k0 + 32 > kvlim);
    if (need_mask) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = k0 + 8 * (r / 4) + 4 * hh + (r % 4);
        if ((CAUSAL && key > qrow) || key >= kvlim) s[x][r] = -INFINITY;
      }
    }
  };

  if (ntiles > 0) {
    const int last = ntiles - 1;
    // Prologue: K_0, V_0 in stage 0, K_1, V_1 in stage 1, then K_2, V_2
    // issued; S^T, dP^T of half-tile (0, 0).
    dma_kv(ktile(0), 0);
    if (last >= 1) dma_kv(ktile(1), 1);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (last >= 2) dma_kv(ktile(2), 2);
    if (nt_w > 0) {
      s[0] = f32x16{};
      dp[0] = negd;
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const int o = tile_slot(lq) * RS + 8 * hh + 16 * kk;
        s[0] = mfma32x16(*(const bf16x8*)(&lds_k[0][o]), qf[kk], s[0]);
        dp[0] = mfma32x16(*(const bf16x8*)(&lds_v[0][o]), gf[kk], dp[0]);
      }
      mask_half(0, ktile(0), 0);
    }
    if constexpr (DROP) {
      gen_begin(ktile(0) * kDqBC);
#pragma unroll
      for (int r = 0; r < 10; ++r) philox_round(kz, drop.k0, drop.k1, r);
      quad_gather(kz);
    }
    // K_j, V_j in stage j % 4.  Tile j waits for K_{j+1}, V_{j+1} (issued
    // two tiles earlier), then issues K_{j+3}, V_{j+3} into the stage of
    // tile j-1.  No fence at the barrier: LDS is only read in the loop, and
    // every read of a stage has returned before its wavefront reaches the
    // barrier after which the stage is refilled.
    for (int j = 0; j < ntiles; ++j) {
      const int kj = ktile(j), kj1 = ktile(j + 1), kj3 = ktile(j + 3);
      if (j + 2 <= last)
        asm volatile("s_waitcnt vmcnt(%0)" :: "n"(kMinBatch) : "memory");
      else
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if (j + 3 <= last) dma_kv(kj3, (j + 3) & 3);
      const int st0 = j & 3, st1 = (j + 1) & 3;
      if (j < nt_w) {
        // step 2j: S^T, dP^T of (j, 1) || dS of (j, 0), dQ += (j, 0)
        step(std::integral_constant<int, 1>{}, st0, 1, st0, 0, kj * kDqBC + 32);
        mask_half(1, kj, 1);
        // step 2j+1: S^T, dP^T of (j+1, 0) || dS of (j, 1), dQ += (j, 1)
        step(std::integral_constant<int, 0>{}, st1, 0, st0, 1, kj1 * kDqBC);
        if (j + 1 < nt_w) mask_half(0, kj1, 0);
      }
    }
  }

  // ---- epilogue: dQ = scale * dQ^T (lane = query, regs = d); with
  // dropout divided by the keep probability.  A lane holds 8-byte pieces of
  // its query's row, so stores straight from the registers would touch 32
  // rows per instruction; instead, once every wavefront is done with the
  // K/V stages, each writes its 32 rows in bf16 to its own area of them
  // (rows padded to D + 8 elements) and reads them back 16 bytes per lane,
  // so that every store instruction writes whole rows.
  const float sq = DROP ? scale / kp : scale;
  constexpr int ES = D + 8;                  // row stride of the area
  constexpr int CPR = D / 8;                 // 16-byte pieces per row
  static_assert(NW * 32 * ES <= 4 * TE, "the rows fit the K stages");
  __syncthreads();
  uint16_t* area = &lds_k[0][0] + w * 32 * ES;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      f32x4 xo;
#pragma unroll
      for (int e = 0; e < 4; ++e) xo[e] = dq_acc[db][4 * g + e] * sq;
      *(bf16x4*)(area + lq * ES + 32 * db + 8 * g + 4 * hh) = to_bf16x4(xo);
    }
  }
#pragma unroll
  for (int i = 0; i < 32 * CPR / 64; ++i) {
    const int row = i * (64 / CPR) + lane / CPR, c = lane % CPR;
    const u32x4 v = *(const u32x4*)(area + row * ES + 8 * c);
    if (qlo + row < N) *(u32x4*)(dQ + head + (size_t)(qlo + row) * D + 8 * c) = v;
  }
}

}  // namespace

int launch_bwd_preprocess(const uint16_t* o, const uint16_t* dO, float* D,
                          int B, int H, int N, int d, hipStream_t stream) {
  const size_t rows = (size_t)B * H * N;
  if (d == 128) {
    constexpr int RPB = kThreads / (128 / 8);
    const dim3 grid((unsigned)((rows + RPB - 1) / RPB));
    hipLaunchKernelGGL(bwd_preprocess_kernel<128>, grid, dim3(kThreads), 0,
                       stream, o, dO, D, rows);
  } else {
    constexpr int RPB = kThreads / (64 / 8);
    const dim3 grid((unsigned)((rows + RPB - 1) / RPB));
    hipLaunchKernelGGL(bwd_preprocess_kernel<64>, grid, dim3(kThreads), 0,
                       stream, o, dO, D, rows);
  }
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

int launch_bwd_dkdv(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                    const uint16_t* dO, const float* lse, const float* D,
                    const uint8_t* block_mask, uint16_t* dk, uint16_t* dv,
                    int B, int H, int N, int d, float scale, int causal,
                    const Dropout* drop, const int32_t* kv_len,
                    hipStream_t stream) {
  if (d != kD && d != 64) return -3;
  if (d != kD && block_mask != nullptr && drop != nullptr) return -3;
  const int n_kblk = (N + kBK - 1) / kBK;
  const float c = (float)((double)scale * 1.4426950408889634);
  // Head dim 128 on grids with at least one 128-key workgroup per CU, and
  // every block-sparse or dropout call: the pipelined kernel (4 wavefronts,
  // K/V in registers); head dim 64 without dropout on such grids or with a
  // block mask: the pipelined kernel at head dim 64; the rest: 8 wavefronts.
  const bool fills = (long long)B * H * n_kblk >= device_cu_count();
  if (d == 64 && drop == nullptr && (fills || block_mask != nullptr)) {
    const dim3 grid((unsigned)(B * H * n_kblk)), block(256);
#define FA_DKDV64(CC, SS)                                                      \
  hipLaunchKernelGGL((bwd_dkdv_pipe_kernel<CC, SS, false, 64>), grid, block, 0, \
                     stream, q, k, v, dO, lse, D, dk, dv, block_mask, H, N,     \
                     n_kblk, c, scale, Dropout{}, kv_len)
    if (block_mask) {
      if (causal) FA_DKDV64(true, true); else FA_DKDV64(false, true);
    } else {
      if (causal) FA_DKDV64(true, false); else FA_DKDV64(false, false);
    }
#undef FA_DKDV64
    return hipGetLastError() == hipSuccess ? 0 : -6;
  }
  if (d == kD && (fills || block_mask != nullptr || drop != nullptr)) {
    const dim3 grid((unsigned)(B * H * n_kblk)), block(256);
#define FA_DKDV_LAUNCH(CC, SS)                                                  \
  hipLaunchKernelGGL((bwd_dkdv_pipe_kernel<CC, SS>), grid, block, 0, stream, q, \
                     k, v, dO, lse, D, dk, dv, block_mask, H, N, n_kblk, c,     \
                     scale, Dropout{}, kv_len)
#define FA_DKDV_DROP(CC)                                                       \
  hipLaunchKernelGGL((bwd_dkdv_pipe_kernel<CC, false, true>), grid, block, 0,  \
                     stream, q, k, v, dO, lse, D, dk, dv, nullptr, H, N,       \
                     n_kblk, c, scale, *drop)
    if (drop) {
      if (causal) FA_DKDV_DROP(true); else FA_DKDV_DROP(false);
    } else if (block_mask) {
      if (causal) FA_DKDV_LAUNCH(true, true); else FA_DKDV_LAUNCH(false, true);
    } else {
      if (causal) FA_DKDV_LAUNCH(true, false); else FA_DKDV_LAUNCH(false, false);
    }
#undef FA_DKDV_LAUNCH
#undef FA_DKDV_DROP
    return hipGetLastError() == hipSuccess ? 0 : -6;
  }
  const dim3 grid((unsigned)(B * H * n_kblk)), block(kBwdThreads);
#define FA_DKDV_PLAIN(DD, CC)                                                  \
  hipLaunchKernelGGL((bwd_dkdv_kernel<DD, CC>), grid, block, 0, stream, q, k,   \
                     v, dO, lse, D, dk, dv, N, n_kblk, c, scale, Dropout{},     \
                     nullptr, H, kv_len)
  if (d == 64 && drop != nullptr) {
    if (causal)
      hipLaunchKernelGGL((bwd_dkdv_kernel<64, true, true>), grid, block, 0,
                         stream, q, k, v, dO, lse, D, dk, dv, N, n_kblk, c,
                         scale, *drop, nullptr, H);
    else
      hipLaunchKernelGGL((bwd_dkdv_kernel<64, false, true>), grid, block, 0,
                         stream, q, k, v, dO, lse, D, dk, dv, N, n_kblk, c,
                         scale, *drop, nullptr, H);
  } else if (d == 64 && block_mask != nullptr) {
    if (causal)
      hipLaunchKernelGGL((bwd_dkdv_kernel<64, true, false, true>), grid, block,
                         0, stream, q, k, v, dO, lse, D, dk, dv, N, n_kblk, c,
                         scale, Dropout{}, block_mask, H);
    else
      hipLaunchKernelGGL((bwd_dkdv_kernel<64, false, false, true>), grid,
                         block, 0, stream, q, k, v, dO, lse, D, dk, dv, N,
                         n_kblk, c, scale, Dropout{}, block_mask, H);
  } else if (d == 64) {
    if (causal) FA_DKDV_PLAIN(64, true); else FA_DKDV_PLAIN(64, false);
  } else {
    if (causal) FA_DKDV_PLAIN(128, true); else FA_DKDV_PLAIN(128, false);
  }
#undef FA_DKDV_PLAIN
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

int launch_bwd_dq(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                  const uint16_t* dO, const float* lse, const float* D,
                  const uint8_t* block_mask, uint16_t* dq, int B, int H, int N,
                  int d, float scale, int causal, const Dropout* drop,
                  const int32_t* kv_len, hipStream_t stream) {
  if (d != kD && d != 64) return -3;
  if (d != kD && block_mask != nullptr && drop != nullptr) return -3;
  const float c = (float)((double)scale * 1.4426950408889634);
  // Head dim 128 on grids with at least one 256-row workgroup per CU, and
  // every block-sparse call (a workgroup is one block-mask row) or dropout
  // call: the pipelined kernel; head dim 64 without dropout on such grids or
  // with a block mask: the pipelined kernel at head dim 64; the rest: 128-row
  // workgroups, two per CU.
  const long long grid256 = (long long)B * H * ((N + kDqPBR - 1) / kDqPBR);
  if (d == 64 && drop == nullptr &&
      (grid256 >= device_cu_count() || block_mask != nullptr)) {
    // head dim 64 on grids that fill the chip, or with a block mask: the
    // pipelined kernel
    const int n_qblk = (N + kDqPBR - 1) / kDqPBR;
    const dim3 grid((unsigned)(B * H * n_qblk)), block(512);
#define FA_DQ64(CC, SS)                                                        \
  hipLaunchKernelGGL((bwd_dq_pipe_kernel<CC, SS, false, 64>), grid, block, 0,   \
                     stream, q, k, v, dO, lse, D, dq, block_mask, H, N, n_qblk, \
                     c, scale, Dropout{}, kv_len)
    if (block_mask) {
      if (causal) FA_DQ64(true, true); else FA_DQ64(false, true);
    } else {
      if (causal) FA_DQ64(true, false); else FA_DQ64(false, false);
    }
#undef FA_DQ64
    return hipGetLastError() == hipSuccess ? 0 : -6;
  }
  if (d == kD && (grid256 >= device_cu_count() || block_mask != nullptr ||
                  drop != nullptr)) {
    const int n_qblk = (N + kDqPBR - 1) / kDqPBR;
    const dim3 grid((unsigned)(B * H * n_qblk)), block(512);
#define FA_DQ_LAUNCH(CC, SS)                                                  \
  hipLaunchKernelGGL((bwd_dq_pipe_kernel<CC, SS>), grid, block, 0, stream, q, \
                     k, v, dO, lse, D, dq, block_mask, H, N, n_qblk, c, scale, \
                     Dropout{}, kv_len)
#define FA_DQ_DROP(CC)                                                        \
  hipLaunchKernelGGL((bwd_dq_pipe_kernel<CC, false, true>), grid, block, 0,   \
                     stream, q, k, v, dO, lse, D, dq, nullptr, H, N, n_qblk,  \
                     c, scale, *drop)
    if (drop) {
      if (causal) FA_DQ_DROP(true); else FA_DQ_DROP(false);
    } else if (block_mask) {
      if (causal) FA_DQ_LAUNCH(true, true); else FA_DQ_LAUNCH(false, true);
    } else {
      if (causal) FA_DQ_LAUNCH(true, false); else FA_DQ_LAUNCH(false, false);
    }
#undef FA_DQ_LAUNCH
#undef FA_DQ_DROP
    return hipGetLastError() == hipSuccess ? 0 : -6;
  }
  const int n_qblk = (N + kDqBR - 1) / kDqBR;
  const dim3 grid((unsigned)(B * H * n_qblk)), block(kThreads);
#define FA_DQ_PLAIN(DD, CC)                                                    \
  hipLaunchKernelGGL((bwd_dq_kernel<DD, CC>), grid, block, 0, stream, q, k, v,  \
                     dO, lse, D, dq, N, n_qblk, c, scale, Dropout{}, nullptr, H, \
                     kv_len)
  if (d == 64 && drop != nullptr) {
    if (causal)
      hipLaunchKernelGGL((bwd_dq_kernel<64, true, true>), grid, block, 0,
                         stream, q, k, v, dO, lse, D, dq, N, n_qblk, c, scale,
                         *drop, nullptr, H);
    else
      hipLaunchKernelGGL((bwd_dq_kernel<64, false, true>), grid, block, 0,
                         stream, q, k, v, dO, lse, D, dq, N, n_qblk, c, scale,
                         *drop, nullptr, H);
  } else if (d == 64 && block_mask != nullptr) {
    if (causal)
      hipLaunchKernelGGL((bwd_dq_kernel<64, true, false, true>), grid, block, 0,
                         stream, q, k, v, dO, lse, D, dq, N, n_qblk, c, scale,
                         Dropout{}, block_mask, H);
    else
      hipLaunchKernelGGL((bwd_dq_kernel<64, false, false, true>), grid, block,
                         0, stream, q, k, v, dO, lse, D, dq, N, n_qblk, c,
                         scale, Dropout{}, block_mask, H);
  } else if (d == 64) {
    if (causal) FA_DQ_PLAIN(64, true); else FA_DQ_PLAIN(64, false);
  } else {
    if (causal) FA_DQ_PLAIN(128, true); else FA_DQ_PLAIN(128, false);
  }
#undef FA_DQ_PLAIN
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // namespace fa
