// Causal linear attention forward of libfa (chunkwise), for gfx950.
//
// Pages cited:
//   [LA2] "Lightning Attention-2: A Free Lunch for Handling Unlimited
//         Sequence Lengths in Large Language Models" (abstract): blocks of
//         the sequence, attention-style computation inside a block and the
//         linear-attention kernel trick (a running K^T V state) between
//         blocks, tiled forward for the GPU.
//   [GLA] "[Paper review] Gated Linear Attention Transformers with
//         Hardware-Efficient Training": linear attention as an RNN with a
//         matrix-valued state; the chunkwise form (recurrence between
//         chunks, parallel work inside a chunk).
//
// What is computed: O = scale * tril(Q K^T) V per (batch, head), with no
// softmax, normalisation, decay or gate.  Chunk t of 64 rows:
//     O_t = scale * ( tril(Q_t K_t^T) V_t + Q_t S_{t-1} ),
//     S_t = S_{t-1} + K_t^T V_t            (S_{-1} = 0, d x d, fp32).
//
// gfx950 mapping.  One workgroup per (batch, head, 32 value columns); the
// value blocks of a head are placed on one XCD so that their repeated reads
// of Q and K hit the same L2.  The workgroup walks the chunks in order
// (the state is a recurrence) with four wavefronts:
//   * wavefronts 0 and 1 own query rows 32w .. 32w + 31 of the chunk:
//     A^T = K_t Q_t^T on v_mfma_f32_32x32x16_bf16 (only key blocks <= the
//     query block), the causal mask on the diagonal block, A^T -> bf16
//     (already the B operand of the next product, as P in the softmax
//     kernels), O^T = V_t^T A^T + S_{t-1}^T Q_t^T, with S_{t-1}^T read from
//     LDS as bf16;
//   * wavefronts 2 and 3 own the state: S^T += V_t^T K_t in fp32 registers
//     (the same V_t^T operand; K_t's columns by transposed LDS reads), then
//     write S_t^T as bf16 to the LDS buffer the next chunk reads.
// Chunks go from HBM to LDS by DMA two chunks ahead through three stages;
// one barrier per chunk orders every producer and consumer.  When heads and
// value blocks leave CUs idle (few heads, long sequences), the chunks of a
// head are split into segments: a first pass writes each segment's
// K^T V sum (fp32) to a workspace, and each segment's workgroup then starts
// from the sum of the states before it.
#include "fa.h"
#include "fa_common.h"
#include "fa_launch.h"

#include <algorithm>
#include <type_traits>

namespace fa {

namespace {

constexpr int kLC = 64;          // rows per chunk
constexpr int kLThreads = 256;   // four wavefronts
constexpr int kVB = 32;          // value columns per workgroup
constexpr int kLS = 3;           // LDS stages of the Q/K/V ring

template <int D>
struct LinTile {
  static constexpr int QST = D + 8;          // Q/K rows: 16-B pad (row reads)
  static constexpr int VST = kVB;            // V rows of 64 B: transposed
                                             // reads conflict-free
  static constexpr int SST = D + 8;          // S^T rows (row reads)
};

// STATE_ONLY: the first pass of a split sequence -- each workgroup sums
// K_t^T V_t over its segment and writes that fp32 state to the workspace
// (no Q, no O).  Otherwise the workgroup produces O for its segment,
// starting from the sum of the previous segments' states (zero for the
// first segment or an unsplit sequence).
// REV: the anti-causal form O_i = scale * sum_{j >= i} (q_i . k_j) v_j that
// the backward needs: chunks are walked from the last to the first, a query
// block sees the key blocks at or after it, the diagonal block keeps keys
// at or after the query, and a segment starts from the states of the
// segments after it.
template <int D, bool STATE_ONLY, bool REV = false>
__global__ __launch_bounds__(kLThreads, 1) void linear_fwd_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
    float* __restrict__ seg_state, int BH, int N, int nseg, int seg_chunks,
    float scale) {
  using T = LinTile<D>;
  constexpr int NVB = D / kVB;
  __shared__ __attribute__((aligned(16))) uint16_t lds_q[kLS][kLC * T::QST];
  __shared__ __attribute__((aligned(16))) uint16_t lds_k[kLS][kLC * T::QST];
  __shared__ __attribute__((aligned(16))) uint16_t lds_v[kLS][kLC * T::VST];
  __shared__ __attribute__((aligned(16))) uint16_t lds_s[2][kVB * T::SST];

  // Workgroup -> (head, value block, segment): workgroups are dispatched
  // round-robin over the 8 XCDs, so id % 8 picks the XCD and every value
  // block of a head gets the same one.
  const int id = blockIdx.x;
  const int xcd = id & 7, rest = id >> 3;
  const int vb = rest % NVB;
  const int seg = (rest / NVB) % nseg;
  const int bh = (rest / NVB / nseg) * 8 + xcd;
  if (bh >= BH) return;
  // no other segment needs the state of the last (first, reversed) one
  if (STATE_ONLY && seg == (REV ? 0 : nseg - 1)) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = wave_id();
  const int lq = lane & 31;
  const int hh = lane >> 5;
  const int r16 = lane & 15;
  const int dsub = (lane >> 4) & 1;
  const size_t head = (size_t)bh * N * D;
  const uint16_t* Qh = Q + head;
  const uint16_t* Kh = K + head;
  const uint16_t* Vh = V + head + kVB * vb;
  const int nchunks_all = (N + kLC - 1) / kLC;
  const int c_begin = seg * seg_chunks;
  const int nchunks = min(seg_chunks, nchunks_all - c_begin);   // this segment
  float* const st_base = seg_state + (size_t)(bh * NVB + vb) * nseg * kVB * D;
  // Chunk processed at step u (in order, or from the segment's last).
  auto chunk_of = [&](int u) -> int {
    return REV ? c_begin + nchunks - 1 - u : c_begin + u;
  };
  // Segments whose states the segment starts from: the earlier ones, or
  // (reversed) the later ones.
  const int sp_begin = REV ? seg + 1 : 0, sp_end = REV ? nseg : seg;

  // ---- chunk loads by LDS DMA (buffer loads that write LDS, 16 bytes per
  // lane): slot p of a stage is 16 bytes of row p / RS; slots that are row
  // padding, and rows >= N (the descriptors end at the head's last row),
  // read zero.  Transfer g of a chunk (Q's, then K's, then V's) is issued
  // by wavefront g % 4.
  constexpr int QRS = T::QST / 8, VRS = T::VST / 8;     // 16-B slots per row
  constexpr int QI = kLC * QRS / 64, VI = kLC * VRS / 64;
  constexpr int NI = 2 * QI + VI;                       // transfers per chunk
  constexpr int kIW = (NI + 3) / 4;
  constexpr int kMinBatch = (STATE_ONLY ? NI - QI : NI) / 4;   // per wavefront
  static_assert(kLC * QRS % 64 == 0 && kLC * VRS % 64 == 0 && kMinBatch < 60,
                "DMA layout");
  constexpr unsigned kOut = 1u << 30;
  const unsigned lq0 = lds_addr(&lds_q[0][0]), lk0 = lds_addr(&lds_k[0][0]);
  const unsigned lv0 = lds_addr(&lds_v[0][0]);
  auto dma = [&](int u) __attribute__((always_inline)) {
    const unsigned st = (unsigned)(u % kLS);
    const int row0 = chunk_of(u) * kLC;
    // descriptors of this chunk's rows (they end at row N - 1)
    const int bytes = min(N - row0, kLC) * D * 2;
    const size_t base = (size_t)row0 * D;
    const auto rq = __builtin_amdgcn_make_buffer_rsrc((void*)(Qh + base), (short)0,
                                                      bytes, 0x00020000);
    const auto rk = __builtin_amdgcn_make_buffer_rsrc((void*)(Kh + base), (short)0,
                                                      bytes, 0x00020000);
    const auto rv = __builtin_amdgcn_make_buffer_rsrc((void*)(Vh + base), (short)0,
                                                      bytes - kVB * vb * 2, 0x00020000);
#pragma unroll
    for (int u = 0; u < kIW; ++u) {
      const int g = w + 4 * u;
      if (g < 2 * QI) {
        if (STATE_ONLY && g < QI) continue;         // no Q in the state pass
        const int gi = g % QI;
        const int p = 64 * gi + lane, row = p / QRS, c = p % QRS;
        const unsigned off = c < D / 8 ? (unsigned)((row * D + 8 * c) * 2) : kOut;
        const unsigned lds = (g < QI ? lq0 : lk0) +
                             st * (unsigned)(kLC * T::QST * 2) + 1024u * gi;
        lds_dma16(g < QI ? rq : rk, lds, off);
      } else if (g < NI) {
        const int gi = g - 2 * QI;
        const int p = 64 * gi + lane, row = p / VRS, c = p % VRS;
        const unsigned off = (unsigned)((row * D + 8 * c) * 2);
        lds_dma16(rv, lv0 + st * (unsigned)(kLC * T::VST * 2) + 1024u * gi, off);
      }
    }
  };

  // V_t^T operand (A: rows = the 32 value columns, contraction = keys) of
  // key block kb, half c: element e is key 32kb + 16c + 8(e/4) + 4hh + e%4.
  auto vt_frag = [&](int b, int kb, int c) __attribute__((always_inline)) -> bf16x8 {
    const int key = 32 * kb + 16 * c + 4 * hh + (r16 >> 2);
    const int col = 16 * dsub + 4 * (r16 & 3);
    return join_bf16(lds_read_tr16(&lds_v[b][key * T::VST + col]),
                     lds_read_tr16(&lds_v[b][(key + 8) * T::VST + col]));
  };

  // The state S^T (value columns x d) of this workgroup: wavefronts 2 and 3
  // own d-blocks of 32; fp32 accumulators, C layout (value column
  // 8(r/4) + 4hh + r%4, d = 32 dt + lq).
  constexpr int NDT = D / 32 / 2;            // d-blocks per state wavefront
  f32x16 sacc[NDT];
#pragma unroll
  for (int i = 0; i < NDT; ++i) sacc[i] = f32x16{};
  // The state entering the segment: zero, or the sum of the previous
  // segments' states (state wavefronts, fp32); as bf16 in the buffer the
  // first chunk reads.
  for (int e = tid; e < kVB * T::SST / 8; e += kLThreads)
    *(u32x4*)(&lds_s[1][8 * e]) = u32x4{0u, 0u, 0u, 0u};
  if (!STATE_ONLY && sp_begin < sp_end && w >= 2) {
#pragma unroll
    for (int i = 0; i < NDT; ++i) {
      const int dt = (w - 2) * NDT + i;
      for (int sp = sp_begin; sp < sp_end; ++sp) {
        const float* src = st_base + (size_t)sp * kVB * D;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          sacc[i][r] += src[(8 * (r / 4) + 4 * hh + (r % 4)) * D + 32 * dt + lq];
      }
    }
  }
  __syncthreads();
  if (!STATE_ONLY && sp_begin < sp_end && w >= 2) {
#pragma unroll
    for (int i = 0; i < NDT; ++i) {
      const int dt = (w - 2) * NDT + i;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        lds_s[1][(8 * (r / 4) + 4 * hh + (r % 4)) * T::SST + 32 * dt + lq] =
            __builtin_bit_cast(uint16_t, (__bf16)sacc[i][r]);
    }
  }

  // Chunk t waits for its own transfers (issued two chunks earlier), then
  // the barrier publishes them and the state chunk t - 1 wrote; the stage
  // refilled after it was last read in chunk t - 1.
  dma(0);
  if (nchunks > 1) dma(1);
  for (int u = 0; u < nchunks; ++u) {
    const int b = u % kLS;
    if (u + 1 < nchunks)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kMinBatch) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (u + 2 < nchunks) dma(u + 2);
    const int sb = u & 1;
    const int r0 = chunk_of(u) * kLC;
    // ---- query block QB (wavefront QB): A^T = K Q^T for the key blocks it
    // sees (kb <= QB; reversed kb >= QB) and the inter-chunk term
    // S_{t-1}^T Q^T, as independent MFMA chains interleaved (a dependent
    // chain would wait out each MFMA's latency), then the mask of the
    // diagonal block, A^T -> bf16 and V_t^T A^T.
    auto query_block = [&](auto qb_tag) __attribute__((always_inline)) {
      constexpr int QB = decltype(qb_tag)::value;
      constexpr int NK = REV ? 2 - QB : QB + 1;   // key blocks seen
      constexpr int KB0 = REV ? QB : 0;           // the first of them
      constexpr int KD = QB - KB0;                // the diagonal one
      const int sr = sb ^ 1;
      f32x16 s[NK], oin = f32x16{};
#pragma unroll
      for (int i = 0; i < NK; ++i) s[i] = f32x16{};
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const bf16x8 qf =
            *(const bf16x8*)(&lds_q[b][(32 * QB + lq) * T::QST + 16 * kk + 8 * hh]);
#pragma unroll
        for (int i = 0; i < NK; ++i)
          s[i] = mfma32x16(
              *(const bf16x8*)(&lds_k[b][(32 * (KB0 + i) + lq) * T::QST + 16 * kk + 8 * hh]),
              qf, s[i]);
        oin = mfma32x16(*(const bf16x8*)(&lds_s[sr][lq * T::SST + 16 * kk + 8 * hh]),
                        qf, oin);
      }
      // mask inside the diagonal block: key 8(r/4) + 4hh + r%4 against
      // query lq (keys after the query hidden; reversed, keys before it).
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 8 * (r / 4) + 4 * hh + (r % 4);
        if (REV ? key < lq : key > lq) s[KD][r] = 0.f;
      }
      f32x16 oacc = f32x16{};
#pragma unroll
      for (int i = 0; i < NK; ++i)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          f32x8 p;
#pragma unroll
          for (int e = 0; e < 8; ++e) p[e] = s[i][8 * c + e];
          oacc = mfma32x16(vt_frag(b, KB0 + i, c), to_bf16x8(p), oacc);
        }
      // ---- store O rows r0 + 32QB + lq, columns 32vb + 8g + 4hh + 0..3.
      const int row = r0 + 32 * QB + lq;
      if (row < N) {
        uint16_t* orow = O + head + (size_t)row * D + kVB * vb;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 x;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            x[e] = (oacc[4 * g + e] + oin[4 * g + e]) * scale;
          *(bf16x4*)(orow + 8 * g + 4 * hh) = to_bf16x4(x);
        }
      }
    };
    if (STATE_ONLY && w < 2) {
      // the state pass computes no output
    } else if (w == 0) {
      query_block(std::integral_constant<int, 0>{});
    } else if (w == 1) {
      query_block(std::integral_constant<int, 1>{});
    } else {
      // ---- state: S^T += V_t^T K_t for the d-blocks of this wavefront
      // (their chains interleaved), then S_t^T -> bf16 into the buffer
      // chunk t + 1 reads.
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const bf16x8 vt = vt_frag(b, kb, c);
          const int key = 32 * kb + 16 * c + 4 * hh + (r16 >> 2);
#pragma unroll
          for (int i = 0; i < NDT; ++i) {
            const int col = 32 * ((w - 2) * NDT + i) + 16 * dsub + 4 * (r16 & 3);
            const bf16x8 kc =
                join_bf16(lds_read_tr16(&lds_k[b][key * T::QST + col]),
                          lds_read_tr16(&lds_k[b][(key + 8) * T::QST + col]));
            sacc[i] = mfma32x16(vt, kc, sacc[i]);
          }
        }
#pragma unroll
      for (int i = 0; i < NDT; ++i) {
        const int dt = (w - 2) * NDT + i;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 x;
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = sacc[i][4 * g + e];
          const bf16x4 y = to_bf16x4(x);
          const i16x4 yi = __builtin_bit_cast(i16x4, y);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            lds_s[sb][(8 * g + 4 * hh + e) * T::SST + 32 * dt + lq] = (uint16_t)yi[e];
        }
      }
    }
  }
  if (STATE_ONLY && w >= 2) {
    float* dst = st_base + (size_t)seg * kVB * D;
#pragma unroll
    for (int i = 0; i < NDT; ++i) {
      const int dt = (w - 2) * NDT + i;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        dst[(8 * (r / 4) + 4 * hh + (r % 4)) * D + 32 * dt + lq] = sacc[i][r];
    }
  }
}

}  // namespace

// Split of a head's chunks into segments (one workgroup each) when the
// heads and value blocks alone leave the chip's CUs idle.  The CU count is
// MI355X's, fixed so that the workspace size (which depends on the split)
// does not depend on which device is current when it is queried.
void linear_split(int B, int H, int N, int d, int& nseg, int& seg_chunks) {
  constexpr int kCUs = 256, kMinSegChunks = 4;
  const long long wgs = (long long)B * H * (d / kVB);
  const int nchunks = (N + kLC - 1) / kLC;
  nseg = 1;
  if (wgs < kCUs)
    nseg = (int)std::min<long long>((kCUs + wgs - 1) / wgs,
                                    std::max(1, nchunks / kMinSegChunks));
  seg_chunks = (nchunks + nseg - 1) / nseg;
  nseg = (nchunks + seg_chunks - 1) / seg_chunks;
}

size_t linear_workspace_bytes(int B, int H, int N, int d) {
  int nseg, seg_chunks;
  linear_split(B, H, N, d, nseg, seg_chunks);
  if (nseg == 1) return 0;
  const size_t bytes = (size_t)B * H * (d / kVB) * nseg * kVB * d * 4;
  return (bytes + 255) & ~(size_t)255;
}

int launch_linear_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                      uint16_t* o, float* ws, int B, int H, int N, int d,
                      float scale, hipStream_t stream) {
  const int BH = B * H;
  const int nvb = d / kVB;
  int nseg, seg_chunks;
  linear_split(B, H, N, d, nseg, seg_chunks);
  const dim3 grid((unsigned)(((BH + 7) / 8) * 8 * nvb * nseg)), block(kLThreads);
#define FA_LIN_LAUNCH(DD, SO)                                                \
  hipLaunchKernelGGL((linear_fwd_kernel<DD, SO>), grid, block, 0, stream, q, \
                     k, v, o, ws, BH, N, nseg, seg_chunks, scale)
  if (d == 128) {
    if (nseg > 1) FA_LIN_LAUNCH(128, true);
    FA_LIN_LAUNCH(128, false);
  } else {
    if (nseg > 1) FA_LIN_LAUNCH(64, true);
    FA_LIN_LAUNCH(64, false);
  }
#undef FA_LIN_LAUNCH
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

// Backward of O = scale * tril(Q K^T) V for the loss <dO, O>, as three
// passes of the chunkwise kernel (the workspace, when the sequence is split,
// is reused by each pass in stream order):
//   dQ_i = scale sum_{j <= i} (dO_i . v_j) k_j   causal, (dO, V, K);
//   dK_j = scale sum_{i >= j} (v_j . dO_i) q_i   reversed, (V, dO, Q);
//   dV_j = scale sum_{i >= j} (k_j . q_i) dO_i   reversed, (K, Q, dO).
int launch_linear_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                      const uint16_t* dO, uint16_t* dq, uint16_t* dk,
                      uint16_t* dv, float* ws, int B, int H, int N, int d,
                      float scale, hipStream_t stream) {
  const int BH = B * H;
  const int nvb = d / kVB;
  int nseg, seg_chunks;
  linear_split(B, H, N, d, nseg, seg_chunks);
  const dim3 grid((unsigned)(((BH + 7) / 8) * 8 * nvb * nseg)), block(kLThreads);
#define FA_LIN_PASS(DD, RR, A, BB, C, OUT)                                        do {                                                                              if (nseg > 1)                                                                     hipLaunchKernelGGL((linear_fwd_kernel<DD, true, RR>), grid, block, 0,                              stream, A, BB, C, OUT, ws, BH, N, nseg, seg_chunks,                             scale);                                                    hipLaunchKernelGGL((linear_fwd_kernel<DD, false, RR>), grid, block, 0,                             stream, A, BB, C, OUT, ws, BH, N, nseg, seg_chunks,                             scale);                                                    } while (0)
  if (d == 128) {
    FA_LIN_PASS(128, false, dO, v, k, dq);
    FA_LIN_PASS(128, true, v, dO, q, dk);
    FA_LIN_PASS(128, true, k, q, dO, dv);
  } else {
    FA_LIN_PASS(64, false, dO, v, k, dq);
    FA_LIN_PASS(64, true, v, dO, q, dk);
    FA_LIN_PASS(64, true, k, q, dO, dv);
  }
#undef FA_LIN_PASS
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // namespace fa
