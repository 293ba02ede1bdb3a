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
// gfx950 mapping (one workgroup = 4 or 8 wavefronts, 32 query rows each):
//   * S^T = K_j Q_i^T on v_mfma_f32_32x32x16_bf16: the accumulator layout
//     puts one query per lane (two lanes per query, one per half-wave), so
//     the row max and row sum are in-lane reductions plus one exchange
//     between half-waves.
//   * O^T += V_j^T P^T on the same instruction: the probabilities of the
//     S^T accumulator are already the B operand (same lane, same key
//     order), and V_j^T is read from the row-major LDS tile with
//     ds_read_b64_tr_b16.
//   * K/V tiles of 64 keys stream HBM -> registers -> LDS, double-buffered:
//     the next tile's global loads are in flight while the current tile is
//     computed.  LDS row strides are padded so the MFMA operand reads are
//     free of bank conflicts.
//   * exp is exp2 with scale*log2(e) folded into one FMA per score.
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
__device__ __forceinline__ void fwd_schedule(int wg, int n_qblk, int BH,
                                             bool causal, int& bh, int& qb) {
  if (causal) {
    qb = n_qblk - 1 - wg / BH;
    bh = wg % BH;
  } else {
    bh = wg / n_qblk;
    qb = wg % n_qblk;
  }
}

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
  fwd_schedule(blockIdx.x, n_qblk, BH, CAUSAL, bh, qb);
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
  fwd_schedule(blockIdx.x, n_qblk, BH, CAUSAL, bh, qb);

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

int launch_fwd_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                    const int32_t* kv_len, uint16_t* o, float* lse, int B,
                    int H, int N, int d, float scale, int causal,
                    hipStream_t stream) {
  // Head dim 128 on grids with at least two 256-row workgroups per CU uses
  // 256-row workgroups of 8 wavefronts: each K/V tile staged in LDS then
  // feeds twice as many query rows.  Everything else uses 128-row
  // workgroups of 4 wavefronts, two per CU.
  constexpr int kCUs = 256;
  const long long wide_grid = (long long)B * H * ((N + 255) / 256);
  const bool wide = d == 128 && wide_grid >= 2 * kCUs;
  const int br = wide ? 256 : 128;
  const int n_qblk = (N + br - 1) / br;
  const dim3 grid((unsigned)(B * H * n_qblk)), block(wide ? 512 : 256);
  const float c = (float)((double)scale * 1.4426950408889634);
  const bool kv = kv_len != nullptr;
#define FA_FWD_LAUNCH(DD, CC, KK)                                              \
  do {                                                                         \
    if (wide)                                                                  \
      hipLaunchKernelGGL((fwd_bf16_kernel<DD, 8, CC, KK>), grid, block, 0,     \
                         stream, q, k, v, o, lse, kv_len, H, N, n_qblk, c);    \
    else                                                                       \
      hipLaunchKernelGGL((fwd_bf16_kernel<DD, 4, CC, KK>), grid, block, 0,     \
                         stream, q, k, v, o, lse, kv_len, H, N, n_qblk, c);    \
  } while (0)
  if (d == 64) {
    if (causal) {
      if (kv) FA_FWD_LAUNCH(64, true, true); else FA_FWD_LAUNCH(64, true, false);
    } else {
      if (kv) FA_FWD_LAUNCH(64, false, true); else FA_FWD_LAUNCH(64, false, false);
    }
  } else {
    if (causal) {
      if (kv) FA_FWD_LAUNCH(128, true, true); else FA_FWD_LAUNCH(128, true, false);
    } else {
      if (kv) FA_FWD_LAUNCH(128, false, true); else FA_FWD_LAUNCH(128, false, false);
    }
  }
#undef FA_FWD_LAUNCH
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
