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
// Tiles are loaded one chunk ahead through registers into two LDS buffers;
// one barrier per chunk orders every producer and consumer.
#include "fa.h"
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

namespace {

constexpr int kLC = 64;          // rows per chunk
constexpr int kLThreads = 256;   // four wavefronts
constexpr int kVB = 32;          // value columns per workgroup

template <int D>
struct LinTile {
  static constexpr int QST = D + 8;          // Q/K rows: 16-B pad (row reads)
  static constexpr int VST = kVB;            // V rows of 64 B: transposed
                                             // reads conflict-free
  static constexpr int SST = D + 8;          // S^T rows (row reads)
  static constexpr int QK_CH = kLC * D / 8;  // 16-B chunks of a Q or K tile
  static constexpr int V_CH = kLC * kVB / 8; // 16-B chunks of a V slice
  static constexpr int QK_PT = QK_CH / kLThreads;
  static_assert(QK_CH % kLThreads == 0 && V_CH == kLThreads, "tile split");
};

template <int D>
__global__ __launch_bounds__(kLThreads, 1) void linear_fwd_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, uint16_t* __restrict__ O, int BH, int N,
    float scale) {
  using T = LinTile<D>;
  constexpr int NVB = D / kVB;
  __shared__ __attribute__((aligned(16))) uint16_t lds_q[2][kLC * T::QST];
  __shared__ __attribute__((aligned(16))) uint16_t lds_k[2][kLC * T::QST];
  __shared__ __attribute__((aligned(16))) uint16_t lds_v[2][kLC * T::VST];
  __shared__ __attribute__((aligned(16))) uint16_t lds_s[2][kVB * T::SST];

  // Workgroup -> (head, value block): workgroups are dispatched round-robin
  // over the 8 XCDs, so id % 8 picks the XCD and every value block of a
  // head gets the same one.
  const int id = blockIdx.x;
  const int xcd = id & 7, rest = id >> 3;
  const int vb = rest % NVB;
  const int bh = (rest / NVB) * 8 + xcd;
  if (bh >= BH) return;

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
  const int nchunks = (N + kLC - 1) / kLC;

  // ---- register-staged loads of chunk t (rows >= N read as zero).
  u32x4 qreg[T::QK_PT], kreg[T::QK_PT], vreg;
  auto load = [&](int t) __attribute__((always_inline)) {
    const int r0 = t * kLC;
#pragma unroll
    for (int i = 0; i < T::QK_PT; ++i) {
      const int c = tid + kLThreads * i;
      const int row = c / (D / 8), col = 8 * (c % (D / 8));
      const bool ok = r0 + row < N;
      const size_t off = (size_t)min(r0 + row, N - 1) * D + col;
      const u32x4 a = *(const u32x4*)(Qh + off);
      const u32x4 b = *(const u32x4*)(Kh + off);
      qreg[i] = ok ? a : u32x4{0u, 0u, 0u, 0u};
      kreg[i] = ok ? b : u32x4{0u, 0u, 0u, 0u};
    }
    const int row = tid / (kVB / 8), col = 8 * (tid % (kVB / 8));
    const u32x4 a = *(const u32x4*)(Vh + (size_t)min(r0 + row, N - 1) * D + col);
    vreg = r0 + row < N ? a : u32x4{0u, 0u, 0u, 0u};
  };
  auto store = [&](int b) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < T::QK_PT; ++i) {
      const int c = tid + kLThreads * i;
      const int row = c / (D / 8), col = 8 * (c % (D / 8));
      *(u32x4*)(&lds_q[b][row * T::QST + col]) = qreg[i];
      *(u32x4*)(&lds_k[b][row * T::QST + col]) = kreg[i];
    }
    const int row = tid / (kVB / 8), col = 8 * (tid % (kVB / 8));
    *(u32x4*)(&lds_v[b][row * T::VST + col]) = vreg;
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
  // S_{-1} = 0 in the buffer the first chunk reads.
  for (int e = tid; e < kVB * T::SST / 8; e += kLThreads)
    *(u32x4*)(&lds_s[1][8 * e]) = u32x4{0u, 0u, 0u, 0u};

  if (nchunks > 0) load(0);
  for (int t = 0; t < nchunks; ++t) {
    const int b = t & 1;
    store(b);
    __syncthreads();
    if (t + 1 < nchunks) load(t + 1);
    const int r0 = t * kLC;
    if (w < 2) {
      // ---- query block qb = w: A^T = K Q^T for key blocks kb <= qb.
      const int qb = w;
      bf16x8 qf[D / 16];
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk)
        qf[kk] = *(const bf16x8*)(&lds_q[b][(32 * qb + lq) * T::QST + 16 * kk + 8 * hh]);
      f32x16 oacc = f32x16{};
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (kb > qb) break;
        f32x16 s = f32x16{};
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
          s = mfma32x16(*(const bf16x8*)(&lds_k[b][(32 * kb + lq) * T::QST + 16 * kk + 8 * hh]),
                        qf[kk], s);
        if (kb == qb) {
          // causal mask inside the diagonal block: key 8(r/4) + 4hh + r%4
          // against query lq.
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (8 * (r / 4) + 4 * hh + (r % 4) > lq) s[r] = 0.f;
        }
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          f32x8 p;
#pragma unroll
          for (int e = 0; e < 8; ++e) p[e] = s[8 * c + e];
          oacc = mfma32x16(vt_frag(b, kb, c), to_bf16x8(p), oacc);
        }
      }
      // ---- inter-chunk term: O^T += S_{t-1}^T Q^T.
      const int sr = b ^ 1;
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk)
        oacc = mfma32x16(*(const bf16x8*)(&lds_s[sr][lq * T::SST + 16 * kk + 8 * hh]),
                         qf[kk], oacc);
      // ---- store O rows r0 + 32qb + lq, columns 32vb + 8g + 4hh + 0..3.
      const int row = r0 + 32 * qb + lq;
      if (row < N) {
        uint16_t* orow = O + head + (size_t)row * D + kVB * vb;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 x;
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = oacc[4 * g + e] * scale;
          *(bf16x4*)(orow + 8 * g + 4 * hh) = to_bf16x4(x);
        }
      }
    } else {
      // ---- state: S^T += V_t^T K_t for d-blocks dt of this wavefront,
      // then S_t^T -> bf16 into the buffer chunk t + 1 reads.
#pragma unroll
      for (int i = 0; i < NDT; ++i) {
        const int dt = (w - 2) * NDT + i;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const int key = 32 * kb + 16 * c + 4 * hh + (r16 >> 2);
            const int col = 32 * dt + 16 * dsub + 4 * (r16 & 3);
            const bf16x8 kc =
                join_bf16(lds_read_tr16(&lds_k[b][key * T::QST + col]),
                          lds_read_tr16(&lds_k[b][(key + 8) * T::QST + col]));
            sacc[i] = mfma32x16(vt_frag(b, kb, c), kc, sacc[i]);
          }
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 x;
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = sacc[i][4 * g + e];
          const bf16x4 y = to_bf16x4(x);
          const i16x4 yi = __builtin_bit_cast(i16x4, y);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            lds_s[b][(8 * g + 4 * hh + e) * T::SST + 32 * dt + lq] = (uint16_t)yi[e];
        }
      }
    }
  }
}

}  // namespace

int launch_linear_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                      uint16_t* o, int B, int H, int N, int d, float scale,
                      hipStream_t stream) {
  const int BH = B * H;
  const int nvb = d / kVB;
  const dim3 grid((unsigned)(((BH + 7) / 8) * 8 * nvb)), block(kLThreads);
  if (d == 128)
    hipLaunchKernelGGL((linear_fwd_kernel<128>), grid, block, 0, stream, q, k,
                       v, o, BH, N, scale);
  else
    hipLaunchKernelGGL((linear_fwd_kernel<64>), grid, block, 0, stream, q, k,
                       v, o, BH, N, scale);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // namespace fa
