/*
 * fa.h -- C ABI of libfa.so: exact IO-aware tiled attention for AMD Instinct
 * MI355X (gfx950), forward and backward.
 *
 * Pages cited (titles as the pages give them):
 *   [MM] "Is a full-day context better than a 10-minute context? Flash
 *        attention and the sequence-length question" (marketmaker.cc blog)
 *   [TW] "Flash-Attention 2 for performance optimisation" (Medium blog)
 *   [ZN] "Paper summary: FlashAttention" (zenn.dev)
 *   [LA2], [GLA]: the linear-attention pages, cited at fa_linear_fwd
 *
 * Operation.  O = softmax(scale * Q K^T) V per (batch, head) ([MM] "Why
 * attention is memory-bound"), computed tile by tile with the online-softmax
 * recurrence so that the N x N score matrix never reaches HBM ([MM] "The
 * Flash Attention algorithm", "Online softmax recurrence"; [ZN] "Proposed
 * method": tiling).  The forward also returns the per-row natural-log
 * log-sum-exp LSE_i = m_i + ln(l_i) ([TW] "Flash Attention 2": one statistic
 * L per row instead of m and l).  The backward recomputes P tile by tile from
 * Q, K and LSE instead of storing it ([MM] "Backward pass: recompute instead
 * of store"; [TW] "Recomputation").
 *
 * Visibility.  Key j is visible to query i iff (causal == 0 or j <= i) and
 * j < kv_len[b] (kv_len absent: N).  With causal != 0, key tiles wholly in
 * the future of a query tile are neither loaded nor computed ([MM] "Causal
 * masking").  A query row with no visible key gets O = 0 and LSE = -inf.
 *
 * Layout.  Q, K, V, O, dO, dQ, dK, dV are contiguous row-major [B, H, N, d]
 * (the (batch, heads, seq, head_dim) shape of [MM] "Integration").  LSE is
 * [B, H, N] float32.  kv_len is int32 [B].  bf16 tensors are passed as raw
 * 16-bit patterns (uint16_t).  Accumulation is float32 throughout.
 *
 * Ownership.  Every pointer except `stream` is a DEVICE pointer owned by the
 * caller.  The library allocates nothing, frees nothing and keeps no mutable
 * global state; it is safe to call from several host threads.  Outputs must
 * not alias inputs.  Outputs are fully overwritten.
 *
 * Execution.  Calls are asynchronous: they validate arguments, enqueue
 * kernels on `stream` (a hipStream_t passed as void*; NULL = the default
 * stream) and return without synchronising.  Device-side faults surface at
 * the caller's next synchronisation.
 *
 * Errors.  Every entry point returns FA_OK (0) or a negative FA_ERR_* code.
 * Argument errors are detected before any HIP call is made (so they are
 * testable without a GPU).  FA_ERR_HIP reports a launch failure
 * (hipGetLastError after the launch).  `scale` is not validated; NaN or Inf
 * inputs propagate.  kv_len values are read on the device, not validated, and
 * clamped to [0, N].  There is no fallback path: an unsupported case is an
 * error, never a silent slower route.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum fa_status {
  FA_OK = 0,
  FA_ERR_NULL = -1,      /* a required pointer is NULL                     */
  FA_ERR_SHAPE = -2,     /* B, H or N <= 0, or B*H*N > 2^31-1              */
  FA_ERR_HEADDIM = -3,   /* d is not 64 or 128                             */
  FA_ERR_ALIGN = -4,     /* a tensor pointer is not 16-byte aligned        */
  FA_ERR_WORKSPACE = -5, /* workspace NULL, too small or not 256-B aligned */
  FA_ERR_HIP = -6,       /* the HIP runtime reported a launch error        */
  FA_ERR_DROPOUT = -7,   /* drop probability outside [0, 255.5/256)       */
  FA_ERR_TOO_LARGE = -8  /* B*H*N beyond the fixed scratch of fa_bwd_noalloc */
};

/* Library version, as 10000*major + 100*minor + patch. */
int fa_version(void);

/* Human-readable text for a status code (never NULL; static storage). */
const char* fa_status_string(int status);

/*
 * Forward, bf16 inputs/outputs, float32 accumulation and LSE.
 *   q, k, v : [B,H,N,d] bf16, read only.
 *   o       : [B,H,N,d] bf16, written.
 *   lse     : [B,H,N] float32, written (natural log).
 *   scale   : multiplies Q K^T (1/sqrt(d) for standard attention).
 *   causal  : nonzero = key j visible to query i only when j <= i.
 * d must be 64 or 128.  Equivalent to fa_fwd_kvlen with kv_len = NULL.
 */
int fa_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
           uint16_t* o, float* lse, int B, int H, int N, int d, float scale,
           int causal, void* stream);

/*
 * Forward with per-sequence key padding: in batch b only keys
 * j < kv_len[b] are visible (for every head).  kv_len is a device int32 [B]
 * array, or NULL for no padding.  All N query rows are produced.
 */
int fa_fwd_kvlen(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                 const int32_t* kv_len, uint16_t* o, float* lse, int B, int H,
                 int N, int d, float scale, int causal, void* stream);

/*
 * Block-sparse forward ([ZN] "Overview": block-sparse FlashAttention, which
 * skips whole blocks of the score matrix by a fixed block mask; the page
 * gives no detail, so the reading is the definition restricted by the mask).
 * The block mask has one byte per FA_SPARSE_BQ query rows x FA_SPARSE_BK
 * keys: key j is visible to query i of head h iff
 *     block_mask[(h * ceil(N/FA_SPARSE_BQ) + i / FA_SPARSE_BQ)
 *                * ceil(N/FA_SPARSE_BK) + j / FA_SPARSE_BK] != 0
 * and (causal == 0 or j <= i); the same mask serves every batch entry.
 *   block_mask : device uint8 [H, ceil(N/256), ceil(N/128)], read only.
 *   other arguments as fa_fwd.
 * A block row is one query workgroup of the forward and dQ kernels and a
 * block column one dK/dV workgroup (two key tiles of the forward); dropped
 * blocks are neither loaded nor computed.  A row with no
 * visible key gets O = 0 and LSE = -inf.
 * Errors as fa_fwd, plus FA_ERR_NULL for a NULL block_mask and FA_ERR_SHAPE
 * when ceil(N/128) exceeds FA_SPARSE_MAX_KEY_BLOCKS (N > 131072).
 */
#define FA_SPARSE_BQ 256
#define FA_SPARSE_BK 128
#define FA_SPARSE_MAX_KEY_BLOCKS 1024
int fa_fwd_block_sparse(const uint16_t* q, const uint16_t* k,
                        const uint16_t* v, const uint8_t* block_mask,
                        uint16_t* o, float* lse, int B, int H, int N, int d,
                        float scale, int causal, void* stream);

/*
 * Forward, float32 inputs and outputs (no reduced precision anywhere):
 * float32 matrix-core products, float32 softmax.  Same shapes and semantics
 * as fa_fwd.
 */
int fa_fwd_f32(const float* q, const float* k, const float* v, float* o,
               float* lse, int B, int H, int N, int d, float scale,
               int causal, void* stream);

/*
 * FP8 forward with incoherent processing ([MM] "FA3: Hopper", item 3: the
 * vectors are rotated at random before block-wise FP8 quantisation, which
 * spreads outliers over all coordinates and lowers the error of FP8
 * attention).  Readings of that passage:
 *   - Rotation: every row of Q and of K is multiplied by R = diag(s) H_d,
 *     s = signs[0..d-1] (+1, or -1 where signs[c] < 0), H_d the
 *     Sylvester-Hadamard matrix, applied in float32 by the fast
 *     Walsh-Hadamard transform, stage t = 0, 1, ... pairing coordinates i
 *     and i + 2^t (bit t of i clear) into (a + b, a - b).  R R^T = d I, so
 *     the scores are taken with scale / d.  V is not rotated.  signs = NULL
 *     skips the rotation (plain FP8) and keeps the scale.
 *   - Block-wise quantisation: every 32 consecutive values (along d for the
 *     rows of Q and K, along the keys for each channel of V; keys past N
 *     are zeros) share a scale 2^e, e the smallest integer with
 *     max|x| <= 448 * 2^e, clamped to [-127, 127]; each value becomes the
 *     OCP E4M3 code of x * 2^-e, rounded to nearest even.  The scale byte
 *     is e + 127 (E8M0).  The matrix cores apply the scales (32-value
 *     blocks are the hardware's scaled-FP8 block).
 *   - Softmax weights are rounded to E4M3 (scale 1) before P V; the row sum
 *     l adds the unrounded float32 weights, so LSE is that of the quantised
 *     scores.  O and LSE as in fa_fwd (bf16 O, float32 natural-log LSE).
 * Head dim 64 or 128; causal or not; no key padding or block mask.
 *
 * Workspace: the quantised operands, in this layout (Np = N rounded up to
 * a multiple of 64, RB = FA_FP8_ROW_BYTES(d)):
 *   Q8 at byte 0:               [B*H][Np][RB]  row n = query n
 *   K8 at byte B*H*Np*RB:       [B*H][Np][RB]  rows permuted in each 64-key
 *                               tile: row 64j + 32t + r8 + 4u + r4 (r8 in
 *                               {0,8,16,24}, u in {0,1}, r4 < 4) holds key
 *                               64j + 32t + 16u + r8/2 + r4
 *   V8 at byte 2*B*H*Np*RB:     [B*H][Np/64][d][80]: channel c of key tile
 *                               j, bytes 0..63 = keys 64j..64j+63, byte 64
 *                               + u = scale of keys 64j+32u .. +31
 * A Q8/K8 row holds the d codes (byte c = coordinate c of the rotated row),
 * then the d/32 scale bytes in the order (u, m) -> byte d + u*(d/64) + m =
 * scale of coordinates 32(2m+u) .. +31, then zeros.  Rows past N are zero.
 */
#define FA_FP8_ROW_BYTES(d) ((d) == 128 ? 144 : 80)
#define FA_FP8_V_ROW_BYTES 80

/* Bytes of workspace the FP8 forward needs (0 for invalid shapes). */
size_t fa_fp8_workspace_size(int B, int H, int N, int d);

/*
 * FP8 step 1: rotate (when signs != NULL) and quantise Q, K and V into the
 * workspace (layout above).  q, k, v: [B,H,N,d] bf16; signs: device int8
 * [d] or NULL; workspace: at least fa_fp8_workspace_size() bytes, 256-byte
 * aligned.  Errors as fa_fwd plus FA_ERR_WORKSPACE.
 */
int fa_fp8_quantize(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                    const int8_t* signs, void* workspace,
                    size_t workspace_bytes, int B, int H, int N, int d,
                    void* stream);

/*
 * FP8 step 2: attention on quantised operands.  score_scale multiplies the
 * dequantised products Q8 K8^T (the caller's scale, divided by d when the
 * operands were rotated).  o: [B,H,N,d] bf16; lse: [B,H,N] float32.
 */
int fa_fwd_fp8_quantized(const void* workspace, size_t workspace_bytes,
                         uint16_t* o, float* lse, int B, int H, int N, int d,
                         float score_scale, int causal, void* stream);

/* Both steps on one stream: fa_fp8_quantize, then fa_fwd_fp8_quantized
 * with scale / d (signs != NULL) or scale (signs == NULL). */
int fa_fwd_fp8(const uint16_t* q, const uint16_t* k, const uint16_t* v,
               const int8_t* signs, uint16_t* o, float* lse, void* workspace,
               size_t workspace_bytes, int B, int H, int N, int d,
               float scale, int causal, void* stream);

/*
 * Causal linear attention, forward ([LA2] "Lightning Attention-2: A Free
 * Lunch for Handling Unlimited Sequence Lengths in Large Language Models",
 * abstract: blocks with attention-style work inside and the linear-attention
 * kernel trick between them; [GLA] "[Paper review] Gated Linear Attention
 * Transformers with Hardware-Efficient Training": the chunkwise form, a
 * recurrence between chunks with a matrix-valued state).  Reading: no
 * softmax, normalisation, decay or gate:
 *     O_i = scale * sum_{j <= i} (q_i . k_j) v_j      (O = scale tril(QK^T) V)
 * computed per 64-row chunk t as scale (tril(Q_t K_t^T) V_t + Q_t S_{t-1})
 * with the state S_t = S_{t-1} + K_t^T V_t kept in float32 and used in bf16.
 *   q, k, v : [B,H,N,d] bf16, read only;  o : [B,H,N,d] bf16, written.
 *   workspace: see fa_linear_workspace_size.
 * d must be 64 or 128.  Errors as fa_fwd, plus FA_ERR_WORKSPACE when a
 * needed workspace is NULL, too small or not 256-byte aligned.
 */
int fa_linear_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                  uint16_t* o, void* workspace, size_t workspace_bytes, int B,
                  int H, int N, int d, float scale, void* stream);

/*
 * Bytes of workspace fa_linear_fwd needs (0 for invalid shapes, and 0 when
 * the sequence is not split: then workspace may be NULL).  When B*H*d/32
 * workgroups would leave CUs idle, the chunks of each head are split into
 * segments; the workspace holds each segment's float32 K^T V state
 * [B*H][d/32][segments][32][d], written by a first pass.  256-byte aligned,
 * owned by the caller, contents on entry irrelevant.
 */
size_t fa_linear_workspace_size(int B, int H, int N, int d);

/*
 * Causal linear attention, backward ([LA2] abstract: the tiled computation
 * serves the backward pass as well as the forward; [GLA] "proposed method":
 * the chunkwise form is what makes training hardware-efficient).  The
 * gradients of <dO, O> for O = scale * tril(Q K^T) V:
 *     dQ_i = scale * sum_{j <= i} (dO_i . v_j) k_j
 *     dK_j = scale * sum_{i >= j} (dO_i . v_j) q_i
 *     dV_j = scale * sum_{i >= j} (q_i . k_j) dO_i
 * dQ is the forward's chunk recurrence on (dO, V, K); dK and dV are the same
 * recurrence walked from the last chunk to the first on (V, dO, Q) and
 * (K, Q, dO), the state then summing the later chunks.  Three passes on one
 * stream; float32 states and accumulation, scores and states rounded to bf16
 * where they enter a matrix product, as in the forward.
 *   q, k, v, dO   : [B,H,N,d] bf16, read only.
 *   dq, dk, dv    : [B,H,N,d] bf16, written (must not alias the inputs).
 *   workspace     : fa_linear_workspace_size(B, H, N, d) bytes (the same
 *                   as the forward's; NULL allowed when that is 0), reused by
 *                   each pass in stream order.
 * d must be 64 or 128.  Errors as fa_linear_fwd.
 */
int fa_linear_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                  const uint16_t* dO, uint16_t* dq, uint16_t* dk, uint16_t* dv,
                  void* workspace, size_t workspace_bytes, int B, int H, int N,
                  int d, float scale, void* stream);

/*
 * The dense backward entry points below take head dimension d = 64 or 128
 * (any other d returns FA_ERR_HEADDIM and fa_bwd_workspace_size returns 0).
 * Grids that fill the chip run the pipelined kernels at either d (at d = 64
 * only without dropout); smaller grids run the 8-wavefront dK/dV and
 * 4-wavefront dQ kernels.  The block-sparse variants always run the
 * pipelined kernels, and so do the dropout variants at d = 128 (at d = 64
 * they run the 8- and 4-wavefront kernels).
 *
 * Bytes of device workspace the backward needs: D [B,H,N] float32 (the row
 * dot products dO_i . O_i), rounded up to 256 bytes.  Returns 0 for invalid
 * shapes.
 */
size_t fa_bwd_workspace_size(int B, int H, int N, int d);

/*
 * Backward of the bf16 forward (no key padding).
 *   q, k, v, o, dO : [B,H,N,d] bf16; o is the forward's output.
 *   lse            : [B,H,N] float32 from the forward.
 *   dq, dk, dv     : [B,H,N,d] bf16, written.
 *   workspace      : device buffer of at least fa_bwd_workspace_size() bytes,
 *                    256-byte aligned, owned by the caller; its contents on
 *                    entry do not matter and are clobbered.
 * P is recomputed tile by tile as exp(scale*Q K^T - LSE).  The gradient is
 * that of <dO, O>:  dV = P^T dO,  dS = P * (dO V^T - D) with
 * D_i = dO_i . O_i,  dQ = scale dS K,  dK = scale dS^T Q.  Accumulation is
 * float32 in registers with no atomics, so results are bitwise
 * reproducible.  Equivalent to fa_bwd_preprocess, fa_bwd_dkdv and fa_bwd_dq
 * in that order on one stream.
 */
int fa_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
           const uint16_t* o, const uint16_t* dO, const float* lse,
           uint16_t* dq, uint16_t* dk, uint16_t* dv, void* workspace,
           size_t workspace_bytes, int B, int H, int N, int d, float scale,
           int causal, void* stream);

/*
 * fa_bwd without a workspace, for callers that cannot allocate device memory
 * (code under stream capture, tight serving loops, harnesses that forbid
 * allocation).  Same arguments, kernels and results as fa_bwd (bitwise); the
 * D rows live in a fixed array of FA_BWD_NOALLOC_MAX_ROWS float32 (8 MiB)
 * that the library holds on every GPU it runs on until the process ends.
 * Its device address is looked up on the first call on each device (the
 * device current at the call, which must be the device of `stream`); no
 * call allocates or frees memory.  Errors as fa_bwd (without
 * FA_ERR_WORKSPACE), plus FA_ERR_TOO_LARGE when B*H*N exceeds
 * FA_BWD_NOALLOC_MAX_ROWS (returned before any HIP call) and FA_ERR_HIP when
 * the array's address cannot be obtained.  All calls on one GPU share the
 * array: calls that overlap on one GPU (streams with no ordering between
 * them) race and must not be issued.
 */
#define FA_BWD_NOALLOC_MAX_ROWS (1 << 21)
int fa_bwd_noalloc(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                   const uint16_t* o, const uint16_t* dO, const float* lse,
                   uint16_t* dq, uint16_t* dk, uint16_t* dv, int B, int H,
                   int N, int d, float scale, int causal, void* stream);

/*
 * Backward of fa_fwd_kvlen (key padding, the BERT-shaped workload): the
 * gradients of fa_bwd with key j of batch entry b visible only while
 * j < kv_len[b] (kv_len device int32 [B], values clamped to [0, N]; NULL
 * means N).  Keys at or past kv_len get dK = dV = 0; a query row with no
 * visible key gets dQ = 0.  o and lse must come from fa_fwd_kvlen with the
 * same kv_len.  Arguments otherwise as fa_bwd; errors as fa_bwd, plus
 * FA_ERR_ALIGN for a kv_len pointer that is not 4-byte aligned.
 */
int fa_bwd_kvlen(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                 const uint16_t* o, const uint16_t* dO, const float* lse,
                 const int32_t* kv_len, uint16_t* dq, uint16_t* dk,
                 uint16_t* dv, void* workspace, size_t workspace_bytes, int B,
                 int H, int N, int d, float scale, int causal, void* stream);

/* Backward stage 1: D_i = dO_i . O_i (float32) into the workspace. */
int fa_bwd_preprocess(const uint16_t* o, const uint16_t* dO, void* workspace,
                      size_t workspace_bytes, int B, int H, int N, int d,
                      void* stream);

/* Backward stage 2: one workgroup per 128-key block (the pipelined kernel:
 * 4 wavefronts, each with its 32 keys' K/V held in registers, on grids with
 * at least one such block per CU; else 8 wavefronts); recomputes S, P, dP
 * and dS per 64-row query tile and writes dK and dV.  Reads D from the
 * workspace. */
int fa_bwd_dkdv(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                const uint16_t* dO, const float* lse, uint16_t* dk,
                uint16_t* dv, const void* workspace, size_t workspace_bytes,
                int B, int H, int N, int d, float scale, int causal,
                void* stream);

/* Backward stage 3: one workgroup per 256-row query block (the pipelined
 * kernel, on grids with at least one such block per CU) or per 128-row
 * query block (otherwise); recomputes S, P, dP and dS per key tile and
 * writes dQ.  Reads D from the workspace. */
int fa_bwd_dq(const uint16_t* q, const uint16_t* k, const uint16_t* v,
              const uint16_t* dO, const float* lse, uint16_t* dq,
              const void* workspace, size_t workspace_bytes, int B, int H,
              int N, int d, float scale, int causal, void* stream);

/*
 * Backward of the block-sparse forward (fa_fwd_block_sparse; [ZN]
 * "Overview"): the same gradients as fa_bwd with P taken over the block
 * mask's visible keys only.
 * dK/dV workgroups (one per 128-key block-mask column) visit only the
 * 64-row query tiles whose block-mask row keeps their column; dQ workgroups
 * (one per 256-row block-mask row) visit only the kept key tiles.  Arguments as fa_bwd plus
 * block_mask as in fa_fwd_block_sparse; lse must come from
 * fa_fwd_block_sparse with the same mask.  d = 64 or 128.  Errors as fa_bwd, plus
 * FA_ERR_NULL for a NULL block_mask and FA_ERR_SHAPE for N > 131072.
 */
int fa_bwd_block_sparse(const uint16_t* q, const uint16_t* k,
                        const uint16_t* v, const uint16_t* o,
                        const uint16_t* dO, const float* lse,
                        const uint8_t* block_mask, uint16_t* dq, uint16_t* dk,
                        uint16_t* dv, void* workspace, size_t workspace_bytes,
                        int B, int H, int N, int d, float scale, int causal,
                        void* stream);

/* Its stages 2 and 3 (after fa_bwd_preprocess), as fa_bwd_dkdv and
 * fa_bwd_dq with the block mask. */
int fa_bwd_dkdv_block_sparse(const uint16_t* q, const uint16_t* k,
                             const uint16_t* v, const uint16_t* dO,
                             const float* lse, const uint8_t* block_mask,
                             uint16_t* dk, uint16_t* dv, const void* workspace,
                             size_t workspace_bytes, int B, int H, int N, int d,
                             float scale, int causal, void* stream);
int fa_bwd_dq_block_sparse(const uint16_t* q, const uint16_t* k,
                           const uint16_t* v, const uint16_t* dO,
                           const float* lse, const uint8_t* block_mask,
                           uint16_t* dq, const void* workspace,
                           size_t workspace_bytes, int B, int H, int N, int d,
                           float scale, int causal, void* stream);

/*
 * Attention with dropout on the weights ([MM] "Integration": the framework
 * call takes a dropout probability next to q, k, v and the causal flag; the
 * pages give nothing more).  O = (P o Z / keep) V with P the softmax of
 * fa_fwd, Z a 0/1 keep mask and keep the keep probability; lse is that of
 * the undropped scores (as fa_fwd), which the backward needs.
 *
 * Random numbers: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel
 * random numbers: as easy as 1, 2, 3", SC 2011).  Element (b, h, i, j) reads
 * byte j % 4 (least significant first) of word i % 4 of the generator
 * output for counter (j / 4, i / 4, b*H + h, offset) and key
 * (seed & 0xFFFFFFFF, seed >> 32); it is kept iff that byte is >= p8, where
 * p8 = round(256 * p_drop) (the drop probability is applied in steps of
 * 1/256), and kept weights are scaled by 256 / (256 - p8).  The mask is a
 * pure function of (seed, offset, p_drop, b, h, i, j): the same arguments
 * give the same mask in the forward and in the backward, on any launch
 * configuration.
 *
 * Arguments as fa_fwd plus p_drop in [0, 255.5/256), seed and offset
 * (callers advance offset, or the seed, between calls that need different
 * masks).  Dense heads only (no key padding or block mask).  Errors as
 * fa_fwd, plus FA_ERR_DROPOUT for p_drop outside that range (or NaN).
 */
int fa_fwd_dropout(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                   uint16_t* o, float* lse, int B, int H, int N, int d,
                   float scale, int causal, float p_drop, uint64_t seed,
                   uint32_t offset, void* stream);

/*
 * Gradients of fa_fwd_dropout for the same mask: dV = (P o Z / keep)^T dO,
 * dP = (dO V^T) o Z / keep, D_i = dO_i . O_i, dS = P o (dP - D),
 * dQ = scale dS K, dK = scale dS^T Q.  Arguments as fa_bwd plus p_drop,
 * seed and offset, which must be those of the forward call that produced o
 * and lse.  d = 64 or 128.  Errors as fa_bwd plus FA_ERR_DROPOUT.
 */
int fa_bwd_dropout(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                   const uint16_t* o, const uint16_t* dO, const float* lse,
                   uint16_t* dq, uint16_t* dk, uint16_t* dv, void* workspace,
                   size_t workspace_bytes, int B, int H, int N, int d,
                   float scale, int causal, float p_drop, uint64_t seed,
                   uint32_t offset, void* stream);

/* Its stages 2 and 3 (after fa_bwd_preprocess), as fa_bwd_dkdv and
 * fa_bwd_dq with dropout. */
int fa_bwd_dkdv_dropout(const uint16_t* q, const uint16_t* k,
                        const uint16_t* v, const uint16_t* dO,
                        const float* lse, uint16_t* dk, uint16_t* dv,
                        const void* workspace, size_t workspace_bytes, int B,
                        int H, int N, int d, float scale, int causal,
                        float p_drop, uint64_t seed, uint32_t offset,
                        void* stream);
int fa_bwd_dq_dropout(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                      const uint16_t* dO, const float* lse, uint16_t* dq,
                      const void* workspace, size_t workspace_bytes, int B,
                      int H, int N, int d, float scale, int causal,
                      float p_drop, uint64_t seed, uint32_t offset,
                      void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
