// Forward kernels of libfa: exact tiled attention with an online softmax on
// gfx950 (CDNA4) matrix cores.
//
// Pages cited (titles as the pages give them):
//   [MM] "Is a full-day context better than a 10-minute context? Flash
//        attention and the sequence-length question" (marketmaker.cc blog)
//   [TW] "Flash-Attention 2 for performance optimisation" (Medium blog)
//   [ZN] "Paper summary: FlashAttention" (zenn.dev)
//
// What is computed ([MM] "The Flash Attention algorithm", "Online softmax
// recurrence"): Q is split into row blocks and K, V into column blocks; for
// each query row the kernel keeps a running maximum m, a running sum l and an
// unnormalised output accumulator O, and when a new key tile raises m it
// rescales l and O by exp(m_old - m_new).  O is divided by l once after the
// last tile (the deferred normalisation of FA2, [MM] "FA2: parallelism",
// item 1; [TW] "Flash Attention 2"), and the natural-log LSE = m + ln l is
// stored per row ([TW] "Flash Attention 2").  Key tiles wholly in the causal
// future are skipped ([MM] "Causal masking").  The grid covers
// (batch, head, query block) ([MM] "FA2: parallelism", item 2), and each
// wavefront owns a distinct slice of the query block and shares the K/V
// tiles, so no reduction crosses wavefronts (item 3; [TW] "Flash Attention 2").
//
// gfx950 mapping, shared by both bf16 kernels below (the 128-row kernel for
// small grids, the software-pipelined 256-row kernel for large ones):
//   * S^T = K_j Q_i^T on v_mfma_f32_32x32x16_bf16: the accumulator layout
//     puts one query per lane (two lanes per query, one per half-wave), so
//     the row statistics are in-lane reductions plus one exchange between
//     half-waves.
//   * O^T += V_j^T P^T on the same instruction: the probabilities of the
//     S^T accumulator are already the B operand (same lane, same key
//     order), and V_j^T is read from the row-major LDS tile with
//     ds_read_b64_tr_b16.
//   * K/V tiles of 64 keys stream HBM -> registers -> LDS (HBM -> LDS by
//     DMA for head dim 128 in the pipelined kernel); the next tiles' loads
//     are in flight while the current tile is computed.  LDS row strides
//     are padded so the MFMA operand reads are free of bank conflicts.
//   * exp is exp2 with scale*log2(e) folded into one FMA per score.
#include "fa.h"
#include "fa_common.h"
#include "fa_launch.h"

#include <type_traits>

namespace fa {

namespace {

constexpr int kBR = 128;   // query rows per workgroup (32 per wavefront)
constexpr int kBC = 64;    // keys per K/V tile
constexpr int kThreads = 256;
// Growth of the running max (log2 units) tolerated before O is rescaled.
constexpr float kRescaleSlack = 8.f;
// Largest per-lane tile sum of weights accepted against a stale reference.
// Small on purpose: it keeps the reference within a few units of the true
// running max, so that a row's dominant weight stays near 1, where its bf16
// rounding error is smallest (a dominant weight of 2^20 would round with
// the full 2^-8 relative error of bf16 and show in near one-hot rows).
constexpr float kSumLimit = 0x1p8f;
// Block-sparse forward: the block mask has one entry per 256 query rows
// (one workgroup of the pipelined kernel) x 64 keys (one key tile), and
// heads have at most 2048 key tiles.
constexpr int kSparseBQ = FA_SPARSE_BQ;
constexpr int kSparseMaxTiles = 2 * FA_SPARSE_MAX_KEY_BLOCKS;
static_assert(FA_SPARSE_BK == 2 * kBC, "a block-mask column is two key tiles");

template <int D, int NW>
struct FwdTile {
  // K rows padded by 16 B: row stride = 4 (mod 64) banks, conflict-free for
  // the 16-row phases of ds_read_b128.
  static constexpr int KST = D + 8;
  // V rows padded so a group of 4 rows x 64 B covers all 64 banks for the
  // transposed 8-byte reads: stride = 64 (mod 256) bytes.
  static constexpr int VST = D + 32;
  static constexpr int KELEMS = kBC * KST;
  static constexpr int VELEMS = kBC * VST;
  static constexpr int CHUNKS = kBC * D / 8;           // 16-byte chunks per tile
  static constexpr int THREADS = 64 * NW;
  static constexpr int CPT = CHUNKS / THREADS;         // chunks per thread
  static constexpr int BR = 32 * NW;                   // query rows per workgroup
};

// Map a workgroup index to (bh, query block): causal grids run the longest
// query blocks (largest index) first so the tail holds the short ones.

template <int D, int NW, bool CAUSAL, bool KVLEN>
__global__ __launch_bounds__(64 * NW, 8 / NW) void fwd_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
    float* __restrict__ LSE, const int32_t* __restrict__ kv_len, int H,
    int N, int n_qblk, float c_log2) {
  using T = FwdTile<D, NW>;
  __shared__ __attribute__((aligned(16))) uint16_t lds_k[2][T::KELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t lds_v[2][T::VELEMS];

  const int BH = gridDim.x / n_qblk;
  int bh, qb;
  block_schedule(blockIdx.x, n_qblk, BH, CAUSAL, bh, qb);
  const int b = bh / H;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = wave_id();   // wave-uniform (scalar register)
  const int lq = lane & 31;     // query column of the accumulator
  const int hh = lane >> 5;     // half-wave
  const int q0 = qb * T::BR;
  const int qrow = q0 + w * 32 + lq;

  int kvlim = N;
  if (KVLEN) kvlim = min(max(kv_len[b], 0), N);
  int kend = kvlim;
  if (CAUSAL) kend = min(kend, q0 + T::BR);
  const int ntiles = kend > 0 ? (kend + kBC - 1) / kBC : 0;

  const size_t head = (size_t)bh * N * D;
  const uint16_t* Qh = Q + head;
  const uint16_t* Kh = K + head;
  const uint16_t* Vh = V + head;

  // Q_i fragment of this lane: query qrow, d = 16*kk + 8*hh + 0..7.
  bf16x8 qf[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    if (qrow < N) {
      qf[kk] = *(const bf16x8*)(Qh + (size_t)qrow * D + 16 * kk + 8 * hh);
    } else {
      qf[kk] = bf16x8{};
    }
  }

  // A negative scale is folded into Q (bf16 negation is exact) so that the
  // softmax below always sees c_log2 >= 0.
  if (c_log2 < 0.f) {
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) qf[kk] = -qf[kk];
    c_log2 = -c_log2;
  }

  // Cooperative tile loads: chunk c = tid + THREADS*r -> row c/(D/8), col
  // 8*(c%(D/8)).  Rows past N read row N-1 (in bounds) and are replaced by
  // zeros with a select; addresses are a wave-uniform tile base plus a 32-bit
  // per-lane offset.
  u32x4 kreg[T::CPT], vreg[T::CPT];
  auto load_tile = [&](int j) {
    const int k0 = j * kBC;
    const uint16_t* kb = Kh + (size_t)k0 * D;
    const uint16_t* vb = Vh + (size_t)k0 * D;
#pragma unroll
    for (int r = 0; r < T::CPT; ++r) {
      const int c = tid + T::THREADS * r;
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
#pragma unroll
    for (int r = 0; r < T::CPT; ++r) {
      const int c = tid + T::THREADS * r;
      const int row = c / (D / 8);
      const int col = 8 * (c % (D / 8));
      *(u32x4*)(&lds_k[buf][row * T::KST + col]) = kreg[r];
      *(u32x4*)(&lds_v[buf][row * T::VST + col]) = vreg[r];
    }
  };

  f32x16 oacc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) oacc[i] = f32x16{};
  float m_run = -INFINITY;   // running max of scale*log2(e)*s
  float l_run = 0.f;         // this half-wave's share of the running sum

  const int qw0 = q0 + 32 * w;         // first query row of this wavefront
  const int qw1 = qw0 + 31;

  if (ntiles > 0) load_tile(0);
  for (int j = 0; j < ntiles; ++j) {
    const int buf = j & 1;
    store_tile(buf);
    __syncthreads();
    // Prefetch the next tile (the last iteration reloads its own tile: an
    // in-bounds load that keeps the loop free of a branch).
    load_tile(min(j + 1, ntiles - 1));

    const int k0 = j * kBC;
    // Tiles wholly in this wavefront's causal future are skipped.
    if (CAUSAL && k0 > qw1) continue;

    // ---- S^T = K_j Q_i^T (keys x queries), two 32-key blocks.
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
      const uint16_t* kp = &lds_k[buf][(32 * kb + lq) * T::KST + 8 * hh];
      bf16x8 a[D / 16];
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) a[kk] = *(const bf16x8*)(kp + 16 * kk);
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) s[kb] = mfma32x16(a[kk], qf[kk], s[kb]);
    }

    // ---- mask: causal diagonal, ragged tail, key padding.
    const bool need_mask =
        (CAUSAL && k0 + kBC - 1 > qw0) || (k0 + kBC > kvlim);
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + 32 * kb + 8 * (r / 4) + 4 * hh + (r % 4);
          const bool hide = (CAUSAL && key > qrow) || key >= kvlim;
          if (hide) s[kb][r] = -INFINITY;
        }
      }
    }

    // ---- online softmax statistics (scaled log2 domain; c_log2 >= 0).
    // The reference max m_run only moves when some lane's tile max exceeds
    // it by more than kRescaleSlack (then every lane moves to its true
    // running max and rescales O and l); otherwise the exponentials are taken
    // against the stale reference and stay below 2^kRescaleSlack.  Exact in
    // exact arithmetic: O and l share the reference, which cancels in O/l.
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = max_halves(mx);
    const float mt = (mx == -INFINITY) ? -INFINITY : mx * c_log2;
    if (__any(mt > m_run + kRescaleSlack)) {
      const float m_new = fmaxf(m_run, mt);
      const float alpha = __builtin_amdgcn_exp2f(
          m_run - ((m_new == -INFINITY) ? 0.f : m_new));
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < D / 32; ++i) oacc[i] *= alpha;
      m_run = m_new;
    }
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;

    // P^T in bf16 for the P V product; l sums the float32 weights (a sum of
    // the bf16-rounded weights would move LSE by up to 2^-9 relative).
    bf16x8 pb[2][2];
    auto probs = [&](auto masked) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          f32x8 p;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float x = s[kb][8 * c + e];
            float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(x, c_log2, -m_use));
            if constexpr (decltype(masked)::value) {
              if (x == -INFINITY) pe = 0.f;
            }
            p[e] = pe;
            l_run += pe;
          }
          pb[kb][c] = to_bf16x8(p);
        }
      }
    };
    if (need_mask) probs(std::true_type{}); else probs(std::false_type{});

    // ---- O^T += V_j^T P^T.  A operand lane (d, hh) element e is
    // V[32kb + 16c + 8(e/4) + 4hh + e%4][d], read with two transposed reads.
    const int r16 = lane & 15;
    const int dsub = (lane >> 4) & 1;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int dcol = 32 * db + 16 * dsub + 4 * (r16 & 3);
      bf16x8 a[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const int key = 32 * kb + 16 * c + 4 * hh + (r16 >> 2);
          a[kb][c] = join_bf16(lds_read_tr16(&lds_v[buf][key * T::VST + dcol]),
                               lds_read_tr16(&lds_v[buf][(key + 8) * T::VST + dcol]));
        }
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int c = 0; c < 2; ++c) oacc[db] = mfma32x16(a[kb][c], pb[kb][c], oacc[db]);
    }
  }

  // ---- epilogue: combine half-wave sums, normalise, store O and LSE.
  const float l_tot = sum_halves(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (qrow < N) {
    uint16_t* orow = O + head + (size_t)qrow * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = oacc[db][4 * g + e] * inv;
        const bf16x4 y = to_bf16x4(x);
        *(bf16x4*)(orow + 32 * db + 8 * g + 4 * hh) = y;
      }
    }
    if (hh == 0) {
      LSE[(size_t)bh * N + qrow] =
          l_tot > 0.f ? (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2
                      : -INFINITY;
    }
  }
}

// ---------------------------------------------------------------------------
// Software-pipelined forward for large grids.  One workgroup = 4 wavefronts
// = 256 query rows; each wavefront owns two 32-row blocks (rows
// q0 + 32w + 0..31 and q0 + 128 + 32w + 0..31, which balances the causal
// work of the wavefronts) and runs them in lockstep, so every K or V operand
// read from LDS feeds one MFMA of each block.  The key axis is walked in
// half-tiles of 32 keys, t = 2j + kb, and each step overlaps three of them:
//   step t:  S_{t+1} = K_{t+1} Q^T  and  O += V_{t-1}^T P_{t-1}^T  on the
//            matrix cores, while the VALU turns S_t into P_t,
// with MFMAs and exponentials interleaved one by one in issue order (a
// wavefront issues in order, so a run of MFMAs would leave its VALU work
// waiting).  Only the masking of S_{t+1} on diagonal, ragged or padded tiles
// and the rare move of the softmax reference sit between steps.  A tile's
// two steps need K_j, K_{j+1}, V_{j-1} and V_j in LDS, so K and V rotate
// through three stages each with one barrier per tile: a stage is
// overwritten two barriers after its last read.  Tile loads are raw buffer
// loads whose descriptor ends at the last key of the head, so keys past N
// read as zero without per-lane selects.  With head dim 128 and one block
// per wavefront (one workgroup per CU, LDS to spare) the tiles go from HBM
// straight into LDS by DMA, through four stages: tile j issues K_{j+3} and
// V_{j+2}, so every transfer has a full tile of compute to land in.

template <int D, int NW, int NB>
struct PipeTile {
  static constexpr int KST = D + 8;    // as FwdTile: conflict-free reads
  static constexpr int VST = D + 32;
  static constexpr int KELEMS = kBC * KST;
  static constexpr int VELEMS = kBC * VST;
  static constexpr int THREADS = 64 * NW;
  static constexpr int BR = 32 * NW * NB;
  static constexpr int CPT = kBC * D / 8 / THREADS;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint16_t* p,
                                                            int bytes) {
  // 0x00020000: raw 32-bit data format (untyped loads), range-checked.
  return __builtin_amdgcn_make_buffer_rsrc((void*)p, (short)0, bytes,
                                           0x00020000);
}

template <int D, int NW, int NB, bool CAUSAL, bool KVLEN, bool SPARSE,
          bool DROP = false>
__global__ __launch_bounds__(64 * NW, (NW == 8 || D == 64) ? 2 : 1) void fwd_bf16_pipe_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
    float* __restrict__ LSE, const int32_t* __restrict__ kv_len,
    const uint8_t* __restrict__ bmask, int H, int N, int n_qblk,
    float c_log2, Dropout drop) {
  using T = PipeTile<D, NW, NB>;
  static_assert(!SPARSE || T::BR == kSparseBQ,
                "a workgroup is one block-mask row");
  // Head dim 128 with one block per wavefront stages K and V by DMA
  // through four LDS stages; the other shapes stage through registers with
  // three (there the register path measured faster).
  constexpr bool DMA = D == 128 && NB == 1;
  constexpr int NS = DMA ? 4 : 3;
  constexpr int LK = NS - 1, LV = NS - 2;   // DMA lookahead of K and V
  __shared__ __attribute__((aligned(16))) uint16_t lds_k[NS][T::KELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t lds_v[NS][T::VELEMS];

  const int BH = gridDim.x / n_qblk;
  int bh, qb;
  block_schedule(blockIdx.x, n_qblk, BH, CAUSAL, bh, qb);
  const int b = bh / H;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = wave_id();
  const int lq = lane & 31;
  const int hh = lane >> 5;
  const int r16 = lane & 15;
  const int dsub = (lane >> 4) & 1;
  const int q0 = qb * T::BR;
  int qlo[NB], qrow[NB];
#pragma unroll
  for (int c = 0; c < NB; ++c) {
    qlo[c] = q0 + 32 * (w + NW * c);
    qrow[c] = qlo[c] + lq;
  }

  int kvlim = N;
  if (KVLEN) kvlim = min(max(kv_len[b], 0), N);
  int kend = kvlim;
  if (CAUSAL) kend = min(kend, q0 + T::BR);
  int ntiles = kend > 0 ? (kend + kBC - 1) / kBC : 0;
  // Tiles this wavefront computes (its block 1 sees the most keys; block 0
  // is masked on the at most two extra tiles).
  int kend_w = kvlim;
  if (CAUSAL) kend_w = min(kend_w, qlo[NB - 1] + 32);
  int nt_w = kend_w > 0 ? (kend_w + kBC - 1) / kBC : 0;

  // ---- block-sparse: the workgroup walks, in order, the key tiles its
  // block-mask row keeps (a list in LDS); ntiles and nt_w then count list
  // entries, so dropped tiles are neither loaded nor computed.
  __shared__ uint32_t tile_list[SPARSE ? kSparseMaxTiles : 1];
  __shared__ int tile_count;
  if constexpr (SPARSE) {
    const int n_mk = (N + FA_SPARSE_BK - 1) / FA_SPARSE_BK;
    const int n_mq = (N + kSparseBQ - 1) / kSparseBQ;
    const uint8_t* mrow = bmask + ((size_t)(bh % H) * n_mq + qb) * n_mk;
    if (w == 0) {
      int cnt = 0;
      for (int base = 0; base < ntiles; base += 64) {
        const int j = base + lane;      // key tile j lies in mask column j/2
        const bool keep = j < ntiles && mrow[j >> 1] != 0;
        const unsigned long long bal = __ballot(keep);
        const int below = __builtin_popcountll(bal & ((1ull << lane) - 1ull));
        if (keep) tile_list[cnt + below] = (unsigned)j;
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
        const bool in = t < ntiles && (int)tile_list[t] < dense_nt_w;
        nt_w += __builtin_popcountll(__ballot(in));
      }
    }
  }
  // Key tile of list position t (clamped to the last; the position itself
  // when dense).  The loops read all the entries a tile needs before its
  // barrier, so the LDS round trips overlap the wait.
  auto entry = [&](int t) -> unsigned {
    if constexpr (SPARSE)
      return __builtin_amdgcn_readfirstlane(tile_list[max(min(t, ntiles - 1), 0)]);
    else
      return (unsigned)t;
  };
  auto key_tile = [](unsigned e) -> int { return (int)e; };

  const size_t head = (size_t)bh * N * D;
  const uint16_t* Qh = Q + head;
  const uint16_t* Kh = K + head;
  const uint16_t* Vh = V + head;

  bf16x8 qf[NB][D / 16];
#pragma unroll
  for (int c = 0; c < NB; ++c)
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
      qf[c][kk] = qrow[c] < N
                      ? *(const bf16x8*)(Qh + (size_t)qrow[c] * D + 16 * kk + 8 * hh)
                      : bf16x8{};
  if (c_log2 < 0.f) {
#pragma unroll
    for (int c = 0; c < NB; ++c)
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) qf[c][kk] = -qf[c][kk];
    c_log2 = -c_log2;
  }
  // A zero scale becomes a tiny positive one: every visible weight is then
  // exp2(0) to fp32 precision and masked scores (-inf) still give 0.
  c_log2 = fmaxf(c_log2, 1e-30f);
  // Q has arrived before any DMA is issued (a wait the compiler can see,
  // so that it places none of its own inside the tile loop).
  if constexpr (DMA) __builtin_amdgcn_s_waitcnt(kWaitVm0);

  // ---- DMA tile loads (global -> LDS): instruction u of wavefront w fills
  // the 1 KB of the (padded) stage at 1024 (w + NW u), 16 bytes per lane;
  // a lane whose 16 bytes are row padding reads out of range.
  constexpr int KCR = T::KST / 8, VCR = T::VST / 8;     // 16-B slots per row
  constexpr int KI = kBC * KCR / 64, VI = kBC * VCR / 64;
  constexpr int KIW = (KI + NW - 1) / NW, VIW = (VI + NW - 1) / NW;
  constexpr int kMinBatch = KI / NW + VI / NW;
  constexpr unsigned kOut = 1u << 30;
  static_assert(!DMA || (kMinBatch < 16 && T::KELEMS % 512 == 0 &&
                         T::VELEMS % 512 == 0), "DMA layout");
  unsigned dk_off[KIW], dv_off[VIW];
#pragma unroll
  for (int u = 0; u < KIW; ++u) {
    const int p = 64 * (w + NW * u) + lane, row = p / KCR, c = p % KCR;
    dk_off[u] = c < D / 8 ? (unsigned)((row * D + 8 * c) * 2) : kOut;
  }
#pragma unroll
  for (int u = 0; u < VIW; ++u) {
    const int p = 64 * (w + NW * u) + lane, row = p / VCR, c = p % VCR;
    dv_off[u] = c < D / 8 ? (unsigned)((row * D + 8 * c) * 2) : kOut;
  }
  const unsigned lds_k0 = lds_addr(&lds_k[0][0]);
  const unsigned lds_v0 = lds_addr(&lds_v[0][0]);
  auto dma_k = [&](int j, int st) {
    const int k0 = j * kBC;
    const auto rs = tile_rsrc(Kh + (size_t)k0 * D, min(N - k0, kBC) * D * 2);
    const unsigned base = lds_k0 + (unsigned)(st * T::KELEMS * 2);
#pragma unroll
    for (int u = 0; u < KIW; ++u)
      if (KI % NW == 0 || w + NW * u < KI)
        lds_dma16(rs, base + 1024u * (w + NW * u), dk_off[u]);
  };
  auto dma_v = [&](int j, int st) {
    const int k0 = j * kBC;
    const auto rs = tile_rsrc(Vh + (size_t)k0 * D, min(N - k0, kBC) * D * 2);
    const unsigned base = lds_v0 + (unsigned)(st * T::VELEMS * 2);
#pragma unroll
    for (int u = 0; u < VIW; ++u)
      if (VI % NW == 0 || w + NW * u < VI)
        lds_dma16(rs, base + 1024u * (w + NW * u), dv_off[u]);
  };

  // ---- tile loads: thread chunk r covers row (tid + 256r) / (D/8).
  unsigned voff[T::CPT];
  int lds_off_k[T::CPT], lds_off_v[T::CPT];
#pragma unroll
  for (int r = 0; r < T::CPT; ++r) {
    const int cidx = tid + T::THREADS * r;
    const int row = cidx / (D / 8);
    const int col = 8 * (cidx % (D / 8));
    voff[r] = (unsigned)((row * D + col) * 2);
    lds_off_k[r] = row * T::KST + col;
    lds_off_v[r] = row * T::VST + col;
  }
  u32x4 kreg[T::CPT], vreg[T::CPT];
  auto load_k = [&](int j) {
    const int k0 = j * kBC;
    const auto rs = tile_rsrc(Kh + (size_t)k0 * D, min(N - k0, kBC) * D * 2);
#pragma unroll
    for (int r = 0; r < T::CPT; ++r)
      kreg[r] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff[r], 0, 0));
  };
  auto load_v = [&](int j) {
    const int k0 = j * kBC;
    const auto rs = tile_rsrc(Vh + (size_t)k0 * D, min(N - k0, kBC) * D * 2);
#pragma unroll
    for (int r = 0; r < T::CPT; ++r)
      vreg[r] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff[r], 0, 0));
  };
  auto store_k = [&](int st) {
#pragma unroll
    for (int r = 0; r < T::CPT; ++r)
      *(u32x4*)(&lds_k[st][lds_off_k[r]]) = kreg[r];
  };
  auto store_v = [&](int st) {
#pragma unroll
    for (int r = 0; r < T::CPT; ++r)
      *(u32x4*)(&lds_v[st][lds_off_v[r]]) = vreg[r];
  };

  f32x16 oacc[NB][D / 32];
#pragma unroll
  for (int c = 0; c < NB; ++c)
#pragma unroll
    for (int i = 0; i < D / 32; ++i) oacc[c][i] = f32x16{};
  float m_ref[NB], m_use[NB], l_run[NB];
#pragma unroll
  for (int c = 0; c < NB; ++c) {
    m_ref[c] = -INFINITY;   // reference max (scaled log2)
    m_use[c] = 0.f;         // m_ref, or 0 while m_ref = -inf
    l_run[c] = 0.f;
  }
  // Per half-tile parity x: S^T (32 keys x 32 queries) of each block, and
  // P^T of each block in bf16 (two 16-key halves).
  f32x16 s[2][NB];
  bf16x8 pb[2][NB][2];
  float tsum[NB];

  // ---- one step.  xs: parity of S_{t+1} (= parity of P_{t-1}); the
  // exponentials take S_t (parity 1 - xs).  stk/kbs: K stage and 32-key
  // half of S_{t+1}; stv/kbv: V stage and half of P_{t-1}.
  // Operand ring.  With one block per wavefront it is carried across steps:
  // the last slots of a step read the first K operands of the next step
  // (nstk, nkbs), so a step never starts by waiting for LDS (two blocks per
  // wavefront leave no registers for it).
  constexpr bool XP = NB == 1;
  constexpr int kPf = XP ? 4 : 3;
  bf16x8 opr[kPf];

  // ---- dropout bytes.  kz[c][m]: for block c, the keep bytes of the
  // exponentials' half-tile, key group m (keys k0 + 8m + 4hh + b, byte b),
  // i.e. register 4m + b of the score accumulator.  Quad lane w makes the
  // generator call of key group w for the quad's four queries; a step
  // computes the bytes of the next step's half-tile (kzn) in its MFMA
  // slots, and takes them over at its start.
  constexpr int kDB = DROP ? NB : 1;
  uint32_t kz[kDB][4], kzn[kDB][4];
  auto gen_begin = [&](int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < kDB; ++c) {
      kzn[c][0] = (uint32_t)(k0 / 4 + 2 * (lq & 3) + hh);
      kzn[c][1] = (uint32_t)(qrow[c] >> 2);
      kzn[c][2] = (uint32_t)bh;
      kzn[c][3] = drop.offset;
    }
  };
  auto gen_round = [&](int r) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < kDB; ++c) philox_round(kzn[c], drop.k0, drop.k1, r);
  };
  auto gen_end = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < kDB; ++c) quad_gather(kzn[c]);
  };
  auto keep = [&](int c, int r) __attribute__((always_inline)) -> bool {
    return drop_keep(kz[c][r / 4], r % 4, drop.p8);
  };

  // ---- operands of a step: operand i < kS is K's 32x16 slice i (S^T =
  // K Q^T), operand kS + pi is V^T's slice pi (O^T += V^T P^T; d-block
  // pi / 2, 16-key half pi % 2), for the K stage / 32-key half (stk, kbs)
  // and the V stage / half (stv, kbv).
  constexpr int kS = D / 16;             // S MFMAs per block
  constexpr int kP = 2 * (D / 32);       // PV MFMAs per block
  constexpr int kN = kS + kP;            // operand reads (each used NB times)
  static_assert(!XP || (kN % kPf == 0 && kPf <= kS), "ring alignment");
  auto fetch_op = [&](int i, int stk, int kbs, int stv, int kbv) -> bf16x8 {
    if (i < kS)
      return *(const bf16x8*)(&lds_k[stk][(32 * kbs + lq) * T::KST + 8 * hh + 16 * i]);
    const int pi = i - kS;
    const int db = pi / 2, h = pi % 2;
    const int dcol = 32 * db + 16 * dsub + 4 * (r16 & 3);
    const int key = 32 * kbv + 16 * h + 4 * hh + (r16 >> 2);
    return join_bf16(lds_read_tr16(&lds_v[stv][key * T::VST + dcol]),
                     lds_read_tr16(&lds_v[stv][(key + 8) * T::VST + dcol]));
  };
  // Operand of MFMA slot k (per block).  With one block per wavefront the S
  // and P V products alternate (S_0, PV_0, S_1, PV_1, ...) so that no MFMA
  // is issued right after one that accumulates into the same registers (a
  // dependent issue waits out the instruction's latency, which is longer
  // than its issue interval); with two blocks the blocks alternate instead.
  static_assert(NB != 1 || kS == kP, "alternating slots");
  auto op_of = [](int k) constexpr -> int {
    return NB == 1 ? ((k & 1) ? kS + (k >> 1) : (k >> 1)) : k;
  };

  auto step = [&](auto xs_tag, int stk, int kbs, int stv, int kbv, int nstk,
                  int nkbs, int nstv, int nkbv, int k0n) {
    constexpr int XS = decltype(xs_tag)::value;
    constexpr int XE = 1 - XS;
    auto fetch = [&](int i) -> bf16x8 { return fetch_op(i, stk, kbs, stv, kbv); };
    auto fetch_next = [&](int i) -> bf16x8 {
      return fetch_op(i, nstk, nkbs, nstv, nkbv);
    };
    bf16x8 op[XP ? 1 : kPf];   // the ring of a step when it is not carried
    if constexpr (!XP) {
#pragma unroll
      for (int k = 0; k < kPf; ++k) op[k] = fetch(op_of(k));
    }
    // The 16 NB exponentials of the step (16 per block, element el -> block
    // el / 16, half (el / 8) % 2, register el % 8) run as a three-stage
    // pipeline across MFMA slots: slot m takes the FMA of one element group,
    // the exp2 of the group before it and the row-sum adds (and, at the end
    // of an 8-element half, the bf16 conversion) of the group before that,
    // so no instruction waits on the one just issued.
    constexpr int kEl = 16 * NB;                    // exponentials
    constexpr int kM = NB * kN;                     // MFMA slots
    constexpr int kG = kEl / kM > 0 ? kEl / kM : 1; // elements per slot
    constexpr int kSlots = kEl / kG;                // slots with VALU work
    float x[kEl], pe[kEl];
    float t[NB][2];
#pragma unroll
    for (int c = 0; c < NB; ++c) t[c][0] = t[c][1] = 0.f;
    auto el_fma = [&](int g) {
#pragma unroll
      for (int u = 0; u < kG; ++u) {
        const int el = g * kG + u, ce = el / 16, h = (el / 8) % 2, e = el % 8;
        x[el] = __builtin_fmaf(s[XE][ce][8 * h + e], c_log2, -m_use[ce]);
      }
    };
    auto el_exp = [&](int g) {
#pragma unroll
      for (int u = 0; u < kG; ++u) pe[g * kG + u] = __builtin_amdgcn_exp2f(x[g * kG + u]);
    };
    auto el_sum = [&](int g) {
#pragma unroll
      for (int u = 0; u < kG; ++u) {
        const int el = g * kG + u, ce = el / 16;
        t[ce][el & 1] += pe[el];
        if (el % 8 == 7) {
          f32x8 v;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            v[e] = pe[el - 7 + e];
            if constexpr (DROP) {
              if (!keep(ce, (el - 7 + e) % 16)) v[e] = 0.f;
            }
          }
          pb[XE][ce][(el / 8) % 2] = to_bf16x8(v);
        }
      }
    };
    if constexpr (DROP) {
#pragma unroll
      for (int c = 0; c < kDB; ++c)
#pragma unroll
        for (int m = 0; m < 4; ++m) kz[c][m] = kzn[c][m];
      gen_begin(k0n);
    }
#pragma unroll
    for (int m = 0; m < kM + 2; ++m) {
      if (m < kM) {
        const int k = m / NB, c = m % NB, i = op_of(k);
        bf16x8 a;
        if constexpr (XP) {
          a = opr[k % kPf];
          if (c == NB - 1)
            opr[k % kPf] = k + kPf < kN ? fetch(op_of(k + kPf))
                                        : fetch_next(op_of(k + kPf - kN));
        } else {
          a = op[k % kPf];
          if (c == NB - 1 && k + kPf < kN) op[k % kPf] = fetch(op_of(k + kPf));
        }
        if (i < kS) {
          s[XS][c] = mfma32x16(a, qf[c][i], i == 0 ? f32x16{} : s[XS][c]);
        } else {
          const int pi = i - kS;
          oacc[c][pi / 2] = mfma32x16(a, pb[XS][c][pi % 2], oacc[c][pi / 2]);
        }
      }
      if (m < kSlots) el_fma(m);
      if (m >= 1 && m - 1 < kSlots) el_exp(m - 1);
      if (m >= 2 && m - 2 < kSlots) el_sum(m - 2);
      if constexpr (DROP) {
        // The ten generator rounds spread over the slots, the exchange last.
        constexpr int kIt = kM + 2;
#pragma unroll
        for (int r = 0; r < 10; ++r)
          if (m == r * (kIt - 1) / 10) gen_round(r);
        if (m == kIt - 1) gen_end();
      }
      // Without a use here the compiler moves the adds to the step's end.
#pragma unroll
      for (int c = 0; c < NB; ++c) asm volatile("" : "+v"(t[c][0]), "+v"(t[c][1]));
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int c = 0; c < NB; ++c) tsum[c] = t[c][0] + t[c][1];
  };

  // ---- P_t of block c recomputed against the current reference.
  auto probs = [&](int xe, int c) __attribute__((always_inline)) {
    float t = 0.f;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      f32x8 p;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = __builtin_amdgcn_exp2f(
            __builtin_fmaf(s[xe][c][8 * h + e], c_log2, -m_use[c]));
        t += p[e];
        if constexpr (DROP) {
          if (!keep(c, 8 * h + e)) p[e] = 0.f;
        }
      }
      pb[xe][c][h] = to_bf16x8(p);
    }
    tsum[c] = t;
  };

  // ---- Reference bookkeeping without a per-step max.  The weights are
  // taken against a reference m_ref that only has to keep them finite and
  // near 1: O and l share it, so it cancels in O / l and in
  // LSE = m_ref + log l.  While every lane's half-tile sum stays below
  // kSumLimit the step is kept.  Otherwise (and on a row's first step,
  // m_ref = -inf) the reference moves to the true running max, O and l are
  // rescaled by exp2(m_ref_old - m_ref_new) as in the online-softmax
  // recurrence, and the step's weights are recomputed.
  auto settle = [&](int xe) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < NB; ++c) {
      asm volatile("" : "+v"(pb[xe][c][0]), "+v"(pb[xe][c][1]), "+v"(tsum[c]));
      if (__builtin_expect(__any(tsum[c] > kSumLimit || m_ref[c] == -INFINITY), 0)) {
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[xe][c][r]);
        mx = max_halves(mx);
        const float mt = (mx == -INFINITY) ? -INFINITY : mx * c_log2;
        const float m_new = fmaxf(m_ref[c], mt);
        const float alpha = __builtin_amdgcn_exp2f(
            m_ref[c] - ((m_new == -INFINITY) ? 0.f : m_new));
        l_run[c] *= alpha;
#pragma unroll
        for (int i = 0; i < D / 32; ++i) oacc[c][i] *= alpha;
        m_ref[c] = m_new;
        m_use[c] = (m_new == -INFINITY) ? 0.f : m_new;
        probs(xe, c);
      }
      l_run[c] += tsum[c];
    }
  };

  // ---- mask half-tile t = 2j + kb (parity x) where needed; e is the
  // list entry of tile j.
  auto mask_half = [&](int x, unsigned e, int kb) {
    const int k0 = key_tile(e) * kBC + 32 * kb;
    bool need[NB], any = false;
#pragma unroll
    for (int c = 0; c < NB; ++c) {
      need[c] = (CAUSAL && k0 + 31 > qlo[c]) || (k0 + 32 > kvlim);
      any = any || need[c];
    }
    if (__builtin_expect(any, 0)) {
      // (k0 made opaque here, so that the compiler does not compute the
      // 16 keys ahead of the branch on every step)
      int kb0 = k0;
      asm volatile("" : "+s"(kb0));
      int key[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) key[r] = kb0 + 8 * (r / 4) + 4 * hh + (r % 4);
#pragma unroll
      for (int c = 0; c < NB; ++c) {
        if (need[c]) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const bool hide = (CAUSAL && key[r] > qrow[c]) || key[r] >= kvlim;
            if (hide) s[x][c][r] = -INFINITY;
          }
        }
      }
    }
  };


  // ---- O += V^T P^T for the last half-tile (no exponentials left).
  auto pv_only = [&](int x, int stv, int kbv) {
#pragma unroll
    for (int pi = 0; pi < 2 * (D / 32); ++pi) {
      const int db = pi / 2, h = pi % 2;
      const int dcol = 32 * db + 16 * dsub + 4 * (r16 & 3);
      const int key = 32 * kbv + 16 * h + 4 * hh + (r16 >> 2);
      const bf16x8 a =
          join_bf16(lds_read_tr16(&lds_v[stv][key * T::VST + dcol]),
                    lds_read_tr16(&lds_v[stv][(key + 8) * T::VST + dcol]));
#pragma unroll
      for (int c = 0; c < NB; ++c) oacc[c][db] = mfma32x16(a, pb[x][c][h], oacc[c][db]);
    }
  };

  if (DMA && ntiles > 0) {
    const int last = ntiles - 1;
    // Stages: K_j and V_j in stage j % NS.  Tile j waits for K_{j+1} and
    // V_j, then issues K_{j+NS-1} and V_{j+NS-2}.
    const unsigned e0 = entry(0), e1 = entry(1), e2 = entry(2);
    dma_k(key_tile(e0), 0);
    if (last >= 1) dma_k(key_tile(e1), 1);
    dma_v(key_tile(e0), 0);
    for (int e = tid; e < T::VELEMS / 8; e += T::THREADS)
      *(u32x4*)(&lds_v[NS - 1][8 * e]) = u32x4{0, 0, 0, 0};
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int c = 0; c < NB; ++c)
#pragma unroll
        for (int h = 0; h < 2; ++h) pb[x][c][h] = bf16x8{};
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if constexpr (NS == 4) {
      if (last >= 2) dma_k(key_tile(e2), 2);
      if (last >= 1) dma_v(key_tile(e1), 1);
    }
    if (nt_w > 0) {
#pragma unroll
      for (int c = 0; c < NB; ++c) {
        s[0][c] = f32x16{};
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
          s[0][c] = mfma32x16(*(const bf16x8*)(&lds_k[0][lq * T::KST + 8 * hh + 16 * kk]),
                              qf[c][kk], s[0][c]);
      }
      mask_half(0, e0, 0);
    }
    if constexpr (DROP) {
      gen_begin(key_tile(e0) * kBC);
#pragma unroll
      for (int r = 0; r < 10; ++r) gen_round(r);
      gen_end();
    }
    if constexpr (XP) {
      // the first step's operands: K_0 half 1, and (zeros) V stage NS - 1
#pragma unroll
      for (int k = 0; k < kPf; ++k) opr[k] = fetch_op(op_of(k), 0, 1, NS - 1, 1);
    }
    // Tile j: wait for K_{j+1} and V_j, barrier, issue the next DMAs.  No
    // fence: LDS is only read in the loop, and every read of a stage has
    // returned before its wavefront reaches the barrier after which the
    // stage is refilled.
    auto top = [&](int j, unsigned ek, unsigned ev) {
      if (NS == 4 && j + 2 <= last)
        asm volatile("s_waitcnt vmcnt(%0)" :: "n"(kMinBatch) : "memory");
      else
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if (j + LK <= last) dma_k(key_tile(ek), (j + LK) % NS);
      if (j + LV <= last) dma_v(key_tile(ev), (j + LV) % NS);
    };
    for (int j = 0; j < nt_w; ++j) {
      const unsigned ej = entry(j), ej1 = entry(j + 1);
      top(j, entry(j + LK), entry(j + LV));
      const int st0 = j % NS, st1 = (j + 1) % NS, stm = (j + NS - 1) % NS;
      const int kj = key_tile(ej) * kBC, kj1 = key_tile(ej1) * kBC;
      step(std::integral_constant<int, 1>{}, st0, 1, stm, 1, st1, 0, st0, 0, kj + 32);
      settle(0);
      mask_half(1, ej, 1);
      step(std::integral_constant<int, 0>{}, st1, 0, st0, 0, st1, 1, st0, 1, kj1);
      settle(1);
      if (j + 1 < nt_w) mask_half(0, ej1, 0);
    }
    if (nt_w > 0) pv_only(1, (nt_w - 1) % NS, 1);
    for (int j = nt_w; j < ntiles; ++j) top(j, entry(j + LK), entry(j + LV));
  } else if (ntiles > 0) {
    const int last = ntiles - 1;
    // Prologue: K_0 in stage 0, zeros in V stage 2 (the V_{-1} that the
    // first step multiplies by P = 0), S_0 (half 0 of tile 0) and its mask;
    // K_1, V_0 in registers for tile 0's stores.
    const unsigned e0 = entry(0), e1 = entry(1);
    load_k(key_tile(e0));
#pragma unroll
    for (int r = 0; r < T::CPT; ++r) vreg[r] = u32x4{0, 0, 0, 0};
    store_v(2);
    store_k(0);
    load_k(key_tile(e1));
    load_v(key_tile(e0));
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int c = 0; c < NB; ++c)
#pragma unroll
        for (int h = 0; h < 2; ++h) pb[x][c][h] = bf16x8{};
    __syncthreads();
    if (nt_w > 0) {
#pragma unroll
      for (int c = 0; c < NB; ++c) {
        s[0][c] = f32x16{};
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
          s[0][c] = mfma32x16(*(const bf16x8*)(&lds_k[0][lq * T::KST + 8 * hh + 16 * kk]),
                              qf[c][kk], s[0][c]);
      }
      mask_half(0, e0, 0);
    }
    if constexpr (DROP) {
      gen_begin(key_tile(e0) * kBC);
#pragma unroll
      for (int r = 0; r < 10; ++r) gen_round(r);
      gen_end();
    }
    if constexpr (XP) {
      // the first step's operands: K_0 half 1, and (zeros) V stage 2
#pragma unroll
      for (int k = 0; k < kPf; ++k) opr[k] = fetch_op(op_of(k), 0, 1, 2, 1);
    }
    // Stages: K_j and V_j in stage j % 3.  Tile j stores K_{j+1} and V_j,
    // then loads K_{j+2} and V_{j+1}.
    int st0 = 0, st1 = 1, stm = 2;   // j % 3, (j+1) % 3, (j-1) % 3
    for (int j = 0; j < ntiles; ++j) {
      const unsigned ej = entry(j), ej1 = entry(j + 1);
      const unsigned ek = entry(min(j + 2, last)), ev = entry(min(j + 1, last));
      store_k(st1);
      store_v(st0);
      __syncthreads();
      load_k(key_tile(ek));
      load_v(key_tile(ev));
      if (__builtin_expect(j < nt_w, 1)) {
        const int kj = key_tile(ej) * kBC, kj1 = key_tile(ej1) * kBC;
        // step 2j: S of (j, half 1) || P of (j, half 0); O += (j-1, half 1)
        step(std::integral_constant<int, 1>{}, st0, 1, stm, 1, st1, 0, st0, 0, kj + 32);
        settle(0);
        mask_half(1, ej, 1);
        // step 2j+1: S of (j+1, half 0) || P of (j, half 1); O += (j, half 0)
        step(std::integral_constant<int, 0>{}, st1, 0, st0, 0, st1, 1, st0, 1, kj1);
        settle(1);
        if (j + 1 < nt_w) mask_half(0, ej1, 0);
      } else if (j == nt_w) {
        pv_only(1, stm, 1);
      }
      const int tmp = stm;
      stm = st0;
      st0 = st1;
      st1 = tmp;
    }
    if (nt_w == ntiles && nt_w > 0) pv_only(1, stm, 1);
  }

  // ---- epilogue: combine half-wave sums, normalise, store O and LSE.  A
  // lane holds 8-byte pieces of its query's row, so stores straight from
  // the registers touch 32 rows per instruction.  With one block per
  // wavefront, once every wavefront is done with the K/V stages, each
  // writes its rows in bf16 to its own area of them (rows padded to D + 8
  // elements) and reads them back 16 bytes per lane, so that every store
  // instruction writes whole rows; with two blocks per wavefront (whose
  // kernels fill the register file) the lanes store their pieces directly.
  constexpr int ES = D + 8;                  // row stride of the area
  constexpr int CPR = D / 8;                 // 16-byte pieces per row
  constexpr int AREA = NW * NB * 32 * ES;
  constexpr bool IN_K = AREA <= NS * T::KELEMS;
  static_assert(NB != 1 || IN_K || AREA <= NS * T::VELEMS,
                "the rows fit the K or V stages");
  if constexpr (NB == 1) __syncthreads();
  uint16_t* area = (IN_K ? &lds_k[0][0] : &lds_v[0][0]) + w * NB * 32 * ES;
#pragma unroll
  for (int c = 0; c < NB; ++c) {
    const float l_tot = sum_halves(l_run[c]);
    float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    // Dropout: kept weights are divided by the keep probability.
    if constexpr (DROP) inv *= 256.f / (float)(256 - drop.p8);
    uint16_t* orow = O + head + (size_t)qrow[c] * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = oacc[c][db][4 * g + e] * inv;
        if constexpr (NB == 1)
          *(bf16x4*)(area + lq * ES + 32 * db + 8 * g + 4 * hh) = to_bf16x4(x);
        else if (qrow[c] < N)
          *(bf16x4*)(orow + 32 * db + 8 * g + 4 * hh) = to_bf16x4(x);
      }
    if (hh == 0 && qrow[c] < N) {
      LSE[(size_t)bh * N + qrow[c]] =
          l_tot > 0.f ? (m_ref[c] + __builtin_amdgcn_logf(l_tot)) * kLn2
                      : -INFINITY;
    }
  }
  if constexpr (NB == 1) {
#pragma unroll
    for (int i = 0; i < 32 * CPR / 64; ++i) {
      const int row = i * (64 / CPR) + lane / CPR, cc = lane % CPR;
      const u32x4 v = *(const u32x4*)(area + row * ES + 8 * cc);
      if (qlo[0] + row < N)
        *(u32x4*)(O + head + (size_t)(qlo[0] + row) * D + 8 * cc) = v;
    }
  }
}

// ---------------------------------------------------------------------------
// float32 forward: v_mfma_f32_32x32x2_f32 (true fp32 products), 32-key tiles.
// The contraction slot (l/32) of the fp32 instruction takes d in two halves:
// slot h, step kk <-> d = kk + (D/2)*h, the same for the K and Q operands.

constexpr int kBC32 = 32;

template <int D>
struct FwdTile32 {
  static constexpr int KST = D + 4;   // floats; 16-B pad
  static constexpr int VST = D;       // V rows read along d: no conflicts
  static constexpr int KELEMS = kBC32 * KST;
  static constexpr int VELEMS = kBC32 * VST;
  static constexpr int CHUNKS = kBC32 * D / 4;      // float4 chunks per tile
  static constexpr int CPT = CHUNKS / kThreads;
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void fwd_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K,
    const float* __restrict__ V, float* __restrict__ O,
    float* __restrict__ LSE, int H, int N, int n_qblk, float c_log2) {
  using T = FwdTile32<D>;
  __shared__ __attribute__((aligned(16))) float lds_k[2][T::KELEMS];
  __shared__ __attribute__((aligned(16))) float lds_v[2][T::VELEMS];

  const int BH = gridDim.x / n_qblk;
  int bh, qb;
  block_schedule(blockIdx.x, n_qblk, BH, CAUSAL, bh, qb);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = wave_id();   // wave-uniform (scalar register)
  const int lq = lane & 31;
  const int hh = lane >> 5;
  const int q0 = qb * kBR;
  const int qrow = q0 + w * 32 + lq;
  int kend = N;
  if (CAUSAL) kend = min(kend, q0 + kBR);
  const int ntiles = (kend + kBC32 - 1) / kBC32;

  const size_t head = (size_t)bh * N * D;
  const float* Qh = Q + head;
  const float* Kh = K + head;
  const float* Vh = V + head;

  float qf[D / 2];
#pragma unroll
  for (int kk = 0; kk < D / 2; kk += 4) {
    f32x4 x = f32x4{0.f, 0.f, 0.f, 0.f};
    if (qrow < N) x = *(const f32x4*)(Qh + (size_t)qrow * D + (D / 2) * hh + kk);
    qf[kk] = x[0];
    qf[kk + 1] = x[1];
    qf[kk + 2] = x[2];
    qf[kk + 3] = x[3];
  }

  f32x4 kreg[T::CPT], vreg[T::CPT];
  auto load_tile = [&](int j) {
#pragma unroll
    for (int r = 0; r < T::CPT; ++r) {
      const int c = tid + kThreads * r;
      const int row = c / (D / 4);
      const int col = 4 * (c % (D / 4));
      const int key = j * kBC32 + row;
      if (key < N) {
        kreg[r] = *(const f32x4*)(Kh + (size_t)key * D + col);
        vreg[r] = *(const f32x4*)(Vh + (size_t)key * D + col);
      } else {
        kreg[r] = f32x4{0.f, 0.f, 0.f, 0.f};
        vreg[r] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int r = 0; r < T::CPT; ++r) {
      const int c = tid + kThreads * r;
      const int row = c / (D / 4);
      const int col = 4 * (c % (D / 4));
      *(f32x4*)(&lds_k[buf][row * T::KST + col]) = kreg[r];
      *(f32x4*)(&lds_v[buf][row * T::VST + col]) = vreg[r];
    }
  };

  f32x16 oacc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) oacc[i] = f32x16{};
  float m_run = -INFINITY;
  float l_run = 0.f;
  const int qw0 = q0 + 32 * w;
  const int qw1 = qw0 + 31;

  if (ntiles > 0) load_tile(0);
  for (int j = 0; j < ntiles; ++j) {
    const int buf = j & 1;
    store_tile(buf);
    __syncthreads();
    if (j + 1 < ntiles) load_tile(j + 1);
    const int k0 = j * kBC32;
    if (CAUSAL && k0 > qw1) continue;

    f32x16 s = f32x16{};
    const float* kp = &lds_k[buf][lq * T::KST + (D / 2) * hh];
#pragma unroll
    for (int kk = 0; kk < D / 2; kk += 4) {
      const f32x4 a = *(const f32x4*)(kp + kk);
      s = mfma32x2f(a[0], qf[kk], s);
      s = mfma32x2f(a[1], qf[kk + 1], s);
      s = mfma32x2f(a[2], qf[kk + 2], s);
      s = mfma32x2f(a[3], qf[kk + 3], s);
    }
    const bool need_mask = (CAUSAL && k0 + kBC32 - 1 > qw0) || (k0 + kBC32 > N);
    if (need_mask) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = k0 + 8 * (r / 4) + 4 * hh + (r % 4);
        if ((CAUSAL && key > qrow) || key >= N) s[r] = -INFINITY;
      }
    }
    // scaled scores, max in the scaled domain (sign of scale irrelevant)
    float mt = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      if (s[r] != -INFINITY) mt = fmaxf(mt, s[r] * c_log2);
    }
    mt = fmaxf(mt, xor32(mt));
    const float m_new = fmaxf(m_run, mt);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_new;
    float lsum = 0.f;
    float p[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      p[r] = s[r] == -INFINITY
                 ? 0.f
                 : __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c_log2, -m_use));
      lsum += p[r];
    }
    l_run = l_run * alpha + lsum;
#pragma unroll
    for (int i = 0; i < D / 32; ++i) oacc[i] *= alpha;
    // O^T += V^T P^T: one instruction per accumulator register r; slot hh
    // holds key 8(r/4) + 4hh + r%4 for both operands.
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 8 * (r / 4) + 4 * hh + (r % 4);
        const float a = lds_v[buf][key * T::VST + 32 * db + lq];
        oacc[db] = mfma32x2f(a, p[r], oacc[db]);
      }
    }
  }

  const float l_tot = l_run + xor32(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (qrow < N) {
    float* orow = O + head + (size_t)qrow * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = oacc[db][4 * g + e] * inv;
        *(f32x4*)(orow + 32 * db + 8 * g + 4 * hh) = x;
      }
    }
    if (hh == 0) {
      LSE[(size_t)bh * N + qrow] =
          l_tot > 0.f ? (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2
                      : -INFINITY;
    }
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// Launchers (argument validation happens in the C-ABI layer before these).

namespace {

template <int D, bool CAUSAL, bool KVLEN, bool SPARSE, bool DROP = false>
void fwd_bf16_dispatch(bool pipe, bool two_blocks, bool narrow, dim3 grid,
                       dim3 block, hipStream_t stream, const uint16_t* q,
                       const uint16_t* k, const uint16_t* v,
                       uint16_t* o, float* lse, const int32_t* kv_len,
                       const uint8_t* bmask, int H, int N, int n_qblk,
                       float c, Dropout drop) {
  // (Dropout keeps one block per wavefront: two would not fit the registers.)
  if constexpr (D == 64 && !DROP) {
    if (pipe && two_blocks) {
      hipLaunchKernelGGL((fwd_bf16_pipe_kernel<D, 4, 2, CAUSAL, KVLEN, SPARSE, DROP>),
                         grid, block, 0, stream, q, k, v, o, lse, kv_len,
                         bmask, H, N, n_qblk, c, drop);
      return;
    }
    if constexpr (!SPARSE) {
      if (pipe && narrow) {
        hipLaunchKernelGGL((fwd_bf16_pipe_kernel<D, 4, 1, CAUSAL, KVLEN, false, false>),
                           grid, block, 0, stream, q, k, v, o, lse, kv_len,
                           bmask, H, N, n_qblk, c, drop);
        return;
      }
    }
  }
  if (pipe || SPARSE || DROP)
    hipLaunchKernelGGL((fwd_bf16_pipe_kernel<D, 8, 1, CAUSAL, KVLEN, SPARSE, DROP>),
                       grid, block, 0, stream, q, k, v, o, lse, kv_len, bmask,
                       H, N, n_qblk, c, drop);
  else if constexpr (!SPARSE && !DROP)
    hipLaunchKernelGGL((fwd_bf16_kernel<D, 4, CAUSAL, KVLEN>), grid, block, 0,
                       stream, q, k, v, o, lse, kv_len, H, N, n_qblk, c);
}

}  // namespace

int launch_fwd_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                    const int32_t* kv_len, const uint8_t* block_mask,
                    uint16_t* o, float* lse, int B, int H, int N, int d,
                    float scale, int causal, const Dropout* drop,
                    hipStream_t stream) {
  // Grids with at least one 256-row workgroup per CU use the pipelined
  // kernel: head dim 64 with 4 wavefronts of two 32-row blocks when there
  // are two such workgroups per CU (two resident per CU), else 4 wavefronts
  // of one block (128-row workgroups, two resident per CU, which spread a
  // grid that fills the chip less than twice more evenly than 8-wavefront
  // ones); head dim 128 with 8 wavefronts of one block (its two blocks
  // would not fit two wavefronts per SIMD).  Smaller grids use the plain
  // kernel with 128-row workgroups, two per CU.  Block-sparse calls always
  // take the pipelined kernel with 8 wavefronts (one 256-row workgroup per
  // block-mask row), and so do calls with dropout.
  const int cus = device_cu_count();
  const bool sparse = block_mask != nullptr;
  const long long grid256 = (long long)B * H * ((N + 255) / 256);
  const bool pipe = sparse || drop != nullptr || grid256 >= cus;
  const bool two_blocks = d == 64 && grid256 >= 2 * cus;
  const bool narrow = d == 64 && pipe && !two_blocks && !sparse && !drop;
  const int br = pipe && !narrow ? 256 : 128;
  const int n_qblk = (N + br - 1) / br;
  const dim3 grid((unsigned)(B * H * n_qblk));
  const dim3 block(pipe && !two_blocks && !narrow ? 512 : 256);
  const float c = (float)((double)scale * 1.4426950408889634);
  const bool kv = kv_len != nullptr;
#define FA_FWD_LAUNCH(DD, CC, KK, SS)                                          \
  fwd_bf16_dispatch<DD, CC, KK, SS>(pipe, two_blocks, narrow, grid, block,    \
                                    stream, q, k, v, o, lse, kv_len,           \
                                    block_mask, H, N, n_qblk, c, Dropout{})
#define FA_FWD_DROP(DD, CC)                                                    \
  fwd_bf16_dispatch<DD, CC, false, false, true>(                               \
      pipe, two_blocks, narrow, grid, block, stream, q, k, v, o, lse, nullptr, \
      nullptr, H, N, n_qblk, c, *drop)
  // Dropout: dense heads without key padding (the C layer checks).
  if (drop) {
    if (d == 64) {
      if (causal) FA_FWD_DROP(64, true); else FA_FWD_DROP(64, false);
    } else {
      if (causal) FA_FWD_DROP(128, true); else FA_FWD_DROP(128, false);
    }
  } else if (d == 64) {
    if (sparse) {
      if (causal) FA_FWD_LAUNCH(64, true, false, true);
      else FA_FWD_LAUNCH(64, false, false, true);
    } else if (causal) {
      if (kv) FA_FWD_LAUNCH(64, true, true, false); else FA_FWD_LAUNCH(64, true, false, false);
    } else {
      if (kv) FA_FWD_LAUNCH(64, false, true, false); else FA_FWD_LAUNCH(64, false, false, false);
    }
  } else {
    if (sparse) {
      if (causal) FA_FWD_LAUNCH(128, true, false, true);
      else FA_FWD_LAUNCH(128, false, false, true);
    } else if (causal) {
      if (kv) FA_FWD_LAUNCH(128, true, true, false); else FA_FWD_LAUNCH(128, true, false, false);
    } else {
      if (kv) FA_FWD_LAUNCH(128, false, true, false); else FA_FWD_LAUNCH(128, false, false, false);
    }
  }
#undef FA_FWD_LAUNCH
#undef FA_FWD_DROP
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

int launch_fwd_f32(const float* q, const float* k, const float* v, float* o,
                   float* lse, int B, int H, int N, int d, float scale,
                   int causal, hipStream_t stream) {
  const int n_qblk = (N + kBR - 1) / kBR;
  const dim3 grid((unsigned)(B * H * n_qblk)), block(kThreads);
  const float c = (float)((double)scale * 1.4426950408889634);
#define FA_FWD32_LAUNCH(DD, CC)                                          \
  hipLaunchKernelGGL((fwd_f32_kernel<DD, CC>), grid, block, 0, stream, q, \
                     k, v, o, lse, H, N, n_qblk, c)
  if (d == 64) {
    if (causal) FA_FWD32_LAUNCH(64, true); else FA_FWD32_LAUNCH(64, false);
  } else {
    if (causal) FA_FWD32_LAUNCH(128, true); else FA_FWD32_LAUNCH(128, false);
  }
#undef FA_FWD32_LAUNCH
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // namespace fa
