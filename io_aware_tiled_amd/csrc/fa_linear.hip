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
//     kernels), O^T = V_t^T A^T + S_{t-1}^T Q_t^T in one accumulator, with
//     S_{t-1} read from LDS as bf16 (transposed reads);
//   * wavefronts 2 and 3 own the state: S^T += V_t^T K_t in fp32 registers
//     (the same V_t^T operand; K_t's columns by transposed LDS reads), then
//     write S_t as bf16 to the LDS buffer the next chunk reads.
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
  static constexpr int SST = kVB + 8;        // S rows (d x value columns),
                                             // read transposed like V; the
                                             // 16-B pad spreads the 8-byte
                                             // writes of 32 rows over the
                                             // banks (64-B rows put them in
                                             // 4 bank groups)
};

// Wait until at most N vector-memory operations of this wavefront are
// outstanding (N a compile-time constant).
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

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
  constexpr int NKK = D / 16;                // contraction slices of d
  __shared__ __attribute__((aligned(16))) uint16_t lds_q[kLS][kLC * T::QST];
  __shared__ __attribute__((aligned(16))) uint16_t lds_k[kLS][kLC * T::QST];
  __shared__ __attribute__((aligned(16))) uint16_t lds_v[kLS][kLC * T::VST];
  __shared__ __attribute__((aligned(16))) uint16_t lds_s[2][D * T::SST];

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
  // read zero.  A chunk of Q (and of K) is QI transfers of 1 KB, V is VI;
  // wavefront w issues transfers w + 4u of each (u < QI / 4, VI / 4), and
  // the QI % 4 remaining Q and K transfers go one each to wavefronts 0, 1,
  // ...  The lane offsets of a wavefront's transfers are the same for
  // every chunk and are computed once.
  constexpr int QRS = T::QST / 8, VRS = T::VST / 8;     // 16-B slots per row
  constexpr int QI = kLC * QRS / 64, VI = kLC * VRS / 64;
  constexpr int QU = QI / 4, QX = QI % 4, VU = VI / 4;
  static_assert(kLC * QRS % 64 == 0 && kLC * VRS % 64 == 0 && VI % 4 == 0 &&
                    2 * QX <= 4 && VRS == D / 8 / NVB,
                "DMA layout");
  constexpr unsigned kOut = 1u << 30;
  auto qk_off = [&](int gi) -> unsigned {
    const int p = 64 * gi + lane, row = p / QRS, c = p % QRS;
    return c < D / 8 ? (unsigned)((row * D + 8 * c) * 2) : kOut;
  };
  unsigned qoff[QU], voff[VU];
#pragma unroll
  for (int u = 0; u < QU; ++u) qoff[u] = qk_off(w + 4 * u);
#pragma unroll
  for (int u = 0; u < VU; ++u) {
    const int p = 64 * (w + 4 * u) + lane;
    voff[u] = (unsigned)(((p / VRS) * D + 8 * (p % VRS)) * 2);
  }
  // the remaining transfer of wavefront w (Q for w < QX, K for the next QX)
  const bool xq = !STATE_ONLY && w < QX, xk = w >= QX && w < 2 * QX;
  const int xgi = 4 * QU + (w < QX ? w : w - QX);
  const unsigned xoff = qk_off(min(xgi, QI - 1));
  const unsigned lq0 = lds_addr(&lds_q[0][0]), lk0 = lds_addr(&lds_k[0][0]);
  const unsigned lv0 = lds_addr(&lds_v[0][0]);
  constexpr unsigned QSB = kLC * T::QST * 2, VSB = kLC * T::VST * 2;
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
    const unsigned qs = lq0 + st * QSB + 1024u * w, ks = lk0 + st * QSB + 1024u * w;
    const unsigned vs = lv0 + st * VSB + 1024u * w;
    if constexpr (!STATE_ONLY) {
#pragma unroll
      for (int i = 0; i < QU; ++i) lds_dma16(rq, qs + 4096u * i, qoff[i]);
    }
#pragma unroll
    for (int i = 0; i < QU; ++i) lds_dma16(rk, ks + 4096u * i, qoff[i]);
#pragma unroll
    for (int i = 0; i < VU; ++i) lds_dma16(rv, vs + 4096u * i, voff[i]);
    if constexpr (QX > 0) {
      if (xq)
        lds_dma16(rq, lq0 + st * QSB + 1024u * xgi, xoff);
      else if (xk)
        lds_dma16(rk, lk0 + st * QSB + 1024u * xgi, xoff);
    }
  };
  // Vector-memory operations this wavefront issues per chunk: its
  // transfers, and (query wavefronts) the 4 stores of its output rows,
  // which are buffer stores whose descriptor ends at the head's last row,
  // so that they are issued for every chunk.
  constexpr int kNT = (STATE_ONLY ? 0 : QU) + QU + VU;
  constexpr int kNS = 4;
  const bool has_x = xq || xk;
  const bool stores = !STATE_ONLY && w < 2;
  // Chunk u's transfers were issued two chunks earlier; after them this
  // wavefront issued chunk u - 2's stores, chunk u + 1's transfers (when
  // there is one) and chunk u - 1's stores.  Wait until only those (or
  // fewer) are outstanding; the counts below never exceed them.
  auto wait_chunk = [&](int u) __attribute__((always_inline)) {
    if (u + 1 >= nchunks) {
      wait_vm<0>();
    } else if (u == 0 || (u == 1 && !stores)) {
      if (has_x) wait_vm<kNT + 1>(); else wait_vm<kNT>();
    } else if (u == 1) {
      if (has_x) wait_vm<kNT + 1 + kNS>(); else wait_vm<kNT + kNS>();
    } else if (stores) {
      if (has_x) wait_vm<kNT + 1 + 2 * kNS>(); else wait_vm<kNT + 2 * kNS>();
    } else {
      if (has_x) wait_vm<kNT + 1>(); else wait_vm<kNT>();
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
  // S^T operand (A: rows = value columns, contraction = d) of slice kk, read
  // transposed from S (d rows of the value columns) in LDS buffer sb:
  // element e is d = 16kk + 8hh + e (the order of a row read of Q).
  auto st_frag = [&](int sb, int kk) __attribute__((always_inline)) -> bf16x8 {
    const int d = 16 * kk + 8 * hh + (r16 >> 2);
    const int col = 16 * dsub + 4 * (r16 & 3);
    return join_bf16(lds_read_tr16(&lds_s[sb][d * T::SST + col]),
                     lds_read_tr16(&lds_s[sb][(d + 4) * T::SST + col]));
  };

  // The state S^T (value columns x d) of this workgroup: wavefronts 2 and 3
  // own d-blocks of 32; fp32 accumulators, C layout (value column
  // 8(r/4) + 4hh + r%4, d = 32 dt + lq).  As bf16 it goes to LDS as S
  // (row d, the value columns), 8 bytes per store.
  constexpr int NDT = D / 32 / 2;            // d-blocks per state wavefront
  f32x16 sacc[NDT];
#pragma unroll
  for (int i = 0; i < NDT; ++i) sacc[i] = f32x16{};
  auto put_state = [&](int sb) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NDT; ++i) {
      const int dt = (w - 2) * NDT + i;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = sacc[i][4 * g + e];
        *(bf16x4*)(&lds_s[sb][(32 * dt + lq) * T::SST + 8 * g + 4 * hh]) = to_bf16x4(x);
      }
    }
  };
  // The state entering the segment: zero, or the sum of the previous
  // segments' states (state wavefronts, fp32); as bf16 in the buffer the
  // first chunk reads.
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
  if constexpr (!STATE_ONLY) {
    if (w >= 2) put_state(1);
  }
  // (the loads above complete before any transfer is issued, so that the
  // vmcnt counts of the loop see only transfers and stores)
  wait_vm<0>();

  // Output rows of the chunk at step u: buffer stores whose descriptor ends
  // at the head's last row, so rows >= N are dropped.
  auto out_rsrc = [&](int u) __attribute__((always_inline)) {
    const int row0 = chunk_of(u) * kLC;
    return __builtin_amdgcn_make_buffer_rsrc(
        (void*)(O + head + (size_t)row0 * D + kVB * vb), (short)0,
        min(N - row0, kLC) * D * 2 - kVB * vb * 2, 0x00020000);
  };

  // Chunk t waits for its own transfers (issued two chunks earlier), then
  // the barrier publishes them and the state chunk t - 1 wrote; the stage
  // refilled after it was last read in chunk t - 1.
  dma(0);
  if (nchunks > 1) dma(1);
  for (int u = 0; u < nchunks; ++u) {
    const int b = u % kLS;
    wait_chunk(u);
    __syncthreads();
    if (u + 2 < nchunks) dma(u + 2);
    const int sb = u & 1;
    // ---- query block QB (wavefront QB): the inter-chunk term S_{t-1}^T
    // Q^T and A^T = K Q^T for the key blocks it sees (kb <= QB; reversed
    // kb >= QB), as independent MFMA chains interleaved (a dependent chain
    // would wait out each MFMA's latency), then the mask of the diagonal
    // block, A^T -> bf16 and V_t^T A^T onto the inter-chunk term.  The
    // operands of slice kk are read from LDS two slices ahead (scheduling
    // barriers keep that order), and V's with the last two slices.
    auto query_block = [&](auto qb_tag) __attribute__((always_inline)) {
      constexpr int QB = decltype(qb_tag)::value;
      constexpr int NK = REV ? 2 - QB : QB + 1;   // key blocks seen
      constexpr int KB0 = REV ? QB : 0;           // the first of them
      constexpr int KD = QB - KB0;                // the diagonal one
      const int sr = sb ^ 1;
      bf16x8 qf[NKK], kf[NK][NKK], sf[NKK], vf[NK][2];
      auto fetch = [&](int kk) __attribute__((always_inline)) {
        qf[kk] = *(const bf16x8*)(&lds_q[b][(32 * QB + lq) * T::QST + 16 * kk + 8 * hh]);
#pragma unroll
        for (int i = 0; i < NK; ++i)
          kf[i][kk] = *(const bf16x8*)(
              &lds_k[b][(32 * (KB0 + i) + lq) * T::QST + 16 * kk + 8 * hh]);
        sf[kk] = st_frag(sr, kk);
      };
      f32x16 s[NK], acc = f32x16{};
#pragma unroll
      for (int i = 0; i < NK; ++i) s[i] = f32x16{};
      fetch(0);
      fetch(1);
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        if (kk + 2 < NKK) fetch(kk + 2);
        if (kk + 2 == NKK) {
#pragma unroll
          for (int i = 0; i < NK; ++i) vf[i][0] = vt_frag(b, KB0 + i, 0);
        }
        if (kk + 1 == NKK) {
#pragma unroll
          for (int i = 0; i < NK; ++i) vf[i][1] = vt_frag(b, KB0 + i, 1);
        }
        __builtin_amdgcn_sched_barrier(0);
        acc = mfma32x16(sf[kk], qf[kk], acc);
#pragma unroll
        for (int i = 0; i < NK; ++i) s[i] = mfma32x16(kf[i][kk], qf[kk], s[i]);
        __builtin_amdgcn_sched_barrier(0);
      }
      // mask inside the diagonal block: key 8(r/4) + 4hh + r%4 against
      // query lq (keys after the query hidden; reversed, keys before it).
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 8 * (r / 4) + 4 * hh + (r % 4);
        if (REV ? key < lq : key > lq) s[KD][r] = 0.f;
      }
#pragma unroll
      for (int i = 0; i < NK; ++i)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          f32x8 p;
#pragma unroll
          for (int e = 0; e < 8; ++e) p[e] = s[i][8 * c + e];
          acc = mfma32x16(vf[i][c], to_bf16x8(p), acc);
        }
      // ---- store O rows 32QB + lq of the chunk, columns 32vb + 8g + 4hh + 0..3.
      const auto ro = out_rsrc(u);
      const unsigned ooff = (unsigned)(((32 * QB + lq) * D + 4 * hh) * 2);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = acc[4 * g + e] * scale;
        __builtin_amdgcn_raw_buffer_store_b64(
            __builtin_bit_cast(u32x2, to_bf16x4(x)), ro, ooff + 16u * g, 0, 0);
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
      // (their chains interleaved), then S_t as bf16 into the buffer chunk
      // t + 1 reads.
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
      if constexpr (!STATE_ONLY) put_state(sb);
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
