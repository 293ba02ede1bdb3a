// C ABI of libfa (declared in include/fa.h): argument validation, workspace
// layout and dispatch to the gfx950 kernels.  Every argument check runs before
// the first HIP call, so argument errors are reported without touching a GPU.
#include "fa.h"

#include <stdint.h>

#include <mutex>

#include "fa_launch.h"

namespace fa {

int device_cu_count() {
  constexpr int kMaxDevices = 64;
  static std::once_flag once[kMaxDevices];
  static int cus[kMaxDevices];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return 256;
  std::call_once(once[dev], [dev] {
    int n = 0;
    cus[dev] = (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount,
                                      dev) == hipSuccess && n > 0) ? n : 256;
  });
  return cus[dev];
}

}  // namespace fa

namespace {

constexpr int kVersion = 10000;   // 1.0.0

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Shape check shared by all entry points: positive extents, a supported head
// dimension, at most 2^31-1 rows (B*H*N) so every grid fits HIP's 32-bit
// workgroup count.
int check_shape(int B, int H, int N, int d) {
  if (B <= 0 || H <= 0 || N <= 0) return FA_ERR_SHAPE;
  const unsigned long long bh = (unsigned long long)B * (unsigned long long)H;
  const unsigned long long rows = bh * (unsigned long long)N;
  if (rows > 0x7fffffffull) return FA_ERR_SHAPE;
  const unsigned long long qblk = bh * (((unsigned long long)N + 127) / 128);
  if (qblk > 0x7fffffffull) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_HEADDIM;
  return FA_OK;
}

// The dense backward takes head dimension 64 or 128 (as the forward).
int check_shape_bwd(int B, int H, int N, int d) { return check_shape(B, H, N, d); }


size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// The backward workspace holds D [B,H,N] float32 only.
size_t ws_bytes(int B, int H, int N) {
  return align256((size_t)B * H * N * sizeof(float));
}

// FP8 forward workspace: Q8 and K8 rows of FA_FP8_ROW_BYTES(d) bytes for
// N rounded up to 64 rows, then V8 tiles of d x 80 bytes per 64 keys.
size_t fp8_ws_bytes(int B, int H, int N, int d) {
  const size_t bh = (size_t)B * H, np = ((size_t)N + 63) / 64 * 64;
  return 2 * bh * np * FA_FP8_ROW_BYTES(d) + bh * (np / 64) * d * FA_FP8_V_ROW_BYTES;
}

// Dropout parameters: p8 = round(256 p) must lie in 0..255.
int make_dropout(float p_drop, uint64_t seed, uint32_t offset,
                 fa::Dropout* out) {
  if (!(p_drop >= 0.f && p_drop < 255.5f / 256.f)) return FA_ERR_DROPOUT;
  const float x = 256.f * p_drop;
  int p8 = (int)x;
  const float frac = x - (float)p8;
  if (frac > 0.5f || (frac == 0.5f && (p8 & 1))) ++p8;   // ties to even
  if (p8 > 255) return FA_ERR_DROPOUT;
  out->k0 = (uint32_t)(seed & 0xFFFFFFFFu);
  out->k1 = (uint32_t)(seed >> 32);
  out->offset = offset;
  out->p8 = p8;
  return FA_OK;
}

int check_workspace(const void* ws, size_t bytes, int B, int H, int N) {
  if (ws == nullptr) return FA_ERR_WORKSPACE;
  if (((uintptr_t)ws & 255u) != 0) return FA_ERR_WORKSPACE;
  if (bytes < ws_bytes(B, H, N)) return FA_ERR_WORKSPACE;
  return FA_OK;
}

}  // namespace

extern "C" {

int fa_version(void) { return kVersion; }

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "FA_OK: success";
    case FA_ERR_NULL: return "FA_ERR_NULL: a required pointer is NULL";
    case FA_ERR_SHAPE:
      return "FA_ERR_SHAPE: B, H or N is not positive, or the problem is too large";
    case FA_ERR_HEADDIM: return "FA_ERR_HEADDIM: head dimension d must be 64 or 128";
    case FA_ERR_ALIGN: return "FA_ERR_ALIGN: a tensor pointer is not 16-byte aligned";
    case FA_ERR_WORKSPACE:
      return "FA_ERR_WORKSPACE: workspace is NULL, not 256-byte aligned or too small";
    case FA_ERR_HIP: return "FA_ERR_HIP: the HIP runtime reported a launch error";
    case FA_ERR_DROPOUT:
      return "FA_ERR_DROPOUT: drop probability must lie in [0, 255.5/256)";
    case FA_ERR_TOO_LARGE:
      return "FA_ERR_TOO_LARGE: B*H*N exceeds the fixed scratch of fa_bwd_noalloc "
             "(FA_BWD_NOALLOC_MAX_ROWS rows)";
    default: return "unknown fa status code";
  }
}

int fa_fwd_kvlen(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                 const int32_t* kv_len, uint16_t* o, float* lse, int B, int H,
                 int N, int d, float scale, int causal, void* stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  int st = check_shape(B, H, N, d);
  if (st != FA_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
      !aligned16(lse) || ((uintptr_t)kv_len & 3u) != 0)
    return FA_ERR_ALIGN;
  return fa::launch_fwd_bf16(q, k, v, kv_len, nullptr, o, lse, B, H, N, d,
                             scale, causal != 0, nullptr, (hipStream_t)stream);
}

int fa_fwd_block_sparse(const uint16_t* q, const uint16_t* k,
                        const uint16_t* v, const uint8_t* block_mask,
                        uint16_t* o, float* lse, int B, int H, int N, int d,
                        float scale, int causal, void* stream) {
  if (!q || !k || !v || !block_mask || !o || !lse) return FA_ERR_NULL;
  int st = check_shape(B, H, N, d);
  if (st != FA_OK) return st;
  if ((N + FA_SPARSE_BK - 1) / FA_SPARSE_BK > FA_SPARSE_MAX_KEY_BLOCKS)
    return FA_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
      !aligned16(lse))
    return FA_ERR_ALIGN;
  return fa::launch_fwd_bf16(q, k, v, nullptr, block_mask, o, lse, B, H, N,
                             d, scale, causal != 0, nullptr, (hipStream_t)stream);
}

int fa_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
           uint16_t* o, float* lse, int B, int H, int N, int d, float scale,
           int causal, void* stream) {
  return fa_fwd_kvlen(q, k, v, nullptr, o, lse, B, H, N, d, scale, causal,
                      stream);
}

int fa_fwd_f32(const float* q, const float* k, const float* v, float* o,
               float* lse, int B, int H, int N, int d, float scale,
               int causal, void* stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  int st = check_shape(B, H, N, d);
  if (st != FA_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
      !aligned16(lse))
    return FA_ERR_ALIGN;
  return fa::launch_fwd_f32(q, k, v, o, lse, B, H, N, d, scale, causal != 0,
                            (hipStream_t)stream);
}

size_t fa_fp8_workspace_size(int B, int H, int N, int d) {
  if (check_shape(B, H, N, d) != FA_OK) return 0;
  return fp8_ws_bytes(B, H, N, d);
}

int fa_fp8_quantize(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                    const int8_t* signs, void* workspace,
                    size_t workspace_bytes, int B, int H, int N, int d,
                    void* stream) {
  if (!q || !k || !v) return FA_ERR_NULL;
  int st = check_shape(B, H, N, d);
  if (st != FA_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v)) return FA_ERR_ALIGN;
  if (!workspace || ((uintptr_t)workspace & 255u) != 0 ||
      workspace_bytes < fp8_ws_bytes(B, H, N, d))
    return FA_ERR_WORKSPACE;
  return fa::launch_fp8_quantize(q, k, v, signs, (uint8_t*)workspace, B, H,
                                 N, d, (hipStream_t)stream);
}

int fa_fwd_fp8_quantized(const void* workspace, size_t workspace_bytes,
                         uint16_t* o, float* lse, int B, int H, int N, int d,
                         float score_scale, int causal, void* stream) {
  if (!o || !lse) return FA_ERR_NULL;
  int st = check_shape(B, H, N, d);
  if (st != FA_OK) return st;
  if (!aligned16(o) || !aligned16(lse)) return FA_ERR_ALIGN;
  if (!workspace || ((uintptr_t)workspace & 255u) != 0 ||
      workspace_bytes < fp8_ws_bytes(B, H, N, d))
    return FA_ERR_WORKSPACE;
  return fa::launch_fwd_fp8((const uint8_t*)workspace, o, lse, B, H, N, d,
                            score_scale, causal != 0, (hipStream_t)stream);
}

int fa_fwd_fp8(const uint16_t* q, const uint16_t* k, const uint16_t* v,
               const int8_t* signs, uint16_t* o, float* lse, void* workspace,
               size_t workspace_bytes, int B, int H, int N, int d,
               float scale, int causal, void* stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  int st = check_shape(B, H, N, d);
  if (st != FA_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
      !aligned16(lse))
    return FA_ERR_ALIGN;
  st = fa_fp8_quantize(q, k, v, signs, workspace, workspace_bytes, B, H, N,
                       d, stream);
  if (st != FA_OK) return st;
  const float score_scale = signs ? scale / (float)d : scale;
  return fa_fwd_fp8_quantized(workspace, workspace_bytes, o, lse, B, H, N, d,
                              score_scale, causal, stream);
}

size_t fa_linear_workspace_size(int B, int H, int N, int d) {
  if (check_shape(B, H, N, d) != FA_OK) return 0;
  return fa::linear_workspace_bytes(B, H, N, d);
}

int fa_linear_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                  uint16_t* o, void* workspace, size_t workspace_bytes, int B,
                  int H, int N, int d, float scale, void* stream) {
  if (!q || !k || !v || !o) return FA_ERR_NULL;
  int st = check_shape(B, H, N, d);
  if (st != FA_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return FA_ERR_ALIGN;
  const size_t need = fa::linear_workspace_bytes(B, H, N, d);
  if (need > 0 && (!workspace || ((uintptr_t)workspace & 255u) != 0 ||
                   workspace_bytes < need))
    return FA_ERR_WORKSPACE;
  return fa::launch_linear_fwd(q, k, v, o, (float*)workspace, B, H, N, d,
                               scale, (hipStream_t)stream);
}

int fa_linear_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                  const uint16_t* dO, uint16_t* dq, uint16_t* dk, uint16_t* dv,
                  void* workspace, size_t workspace_bytes, int B, int H, int N,
                  int d, float scale, void* stream) {
  if (!q || !k || !v || !dO || !dq || !dk || !dv) return FA_ERR_NULL;
  int st = check_shape(B, H, N, d);
  if (st != FA_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dO) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return FA_ERR_ALIGN;
  const size_t need = fa::linear_workspace_bytes(B, H, N, d);
  if (need > 0 && (!workspace || ((uintptr_t)workspace & 255u) != 0 ||
                   workspace_bytes < need))
    return FA_ERR_WORKSPACE;
  return fa::launch_linear_bwd(q, k, v, dO, dq, dk, dv, (float*)workspace, B,
                               H, N, d, scale, (hipStream_t)stream);
}

size_t fa_bwd_workspace_size(int B, int H, int N, int d) {
  if (check_shape_bwd(B, H, N, d) != FA_OK) return 0;
  return ws_bytes(B, H, N);
}

int fa_bwd_preprocess(const uint16_t* o, const uint16_t* dO, void* workspace,
                      size_t workspace_bytes, int B, int H, int N, int d,
                      void* stream) {
  if (!o || !dO) return FA_ERR_NULL;
  int st = check_shape_bwd(B, H, N, d);
  if (st != FA_OK) return st;
  if (!aligned16(o) || !aligned16(dO)) return FA_ERR_ALIGN;
  st = check_workspace(workspace, workspace_bytes, B, H, N);
  if (st != FA_OK) return st;
  return fa::launch_bwd_preprocess(o, dO, (float*)workspace, B, H, N, d,
                                   (hipStream_t)stream);
}

int fa_bwd_dkdv(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                const uint16_t* dO, const float* lse, uint16_t* dk,
                uint16_t* dv, const void* workspace, size_t workspace_bytes,
                int B, int H, int N, int d, float scale, int causal,
                void* stream) {
  if (!q || !k || !v || !dO || !lse || !dk || !dv) return FA_ERR_NULL;
  int st = check_shape_bwd(B, H, N, d);
  if (st != FA_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dO) ||
      !aligned16(lse) || !aligned16(dk) || !aligned16(dv))
    return FA_ERR_ALIGN;
  st = check_workspace(workspace, workspace_bytes, B, H, N);
  if (st != FA_OK) return st;
  return fa::launch_bwd_dkdv(q, k, v, dO, lse, (const float*)workspace,
                             nullptr, dk, dv, B, H, N, d, scale, causal != 0,
                             nullptr, nullptr, (hipStream_t)stream);
}

int fa_bwd_dq(const uint16_t* q, const uint16_t* k, const uint16_t* v,
              const uint16_t* dO, const float* lse, uint16_t* dq,
              const void* workspace, size_t workspace_bytes, int B, int H,
              int N, int d, float scale, int causal, void* stream) {
  if (!q || !k || !v || !dO || !lse || !dq) return FA_ERR_NULL;
  int st = check_shape_bwd(B, H, N, d);
  if (st != FA_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dO) ||
      !aligned16(lse) || !aligned16(dq))
    return FA_ERR_ALIGN;
  st = check_workspace(workspace, workspace_bytes, B, H, N);
  if (st != FA_OK) return st;
  return fa::launch_bwd_dq(q, k, v, dO, lse, (const float*)workspace, nullptr,
                           dq, B, H, N, d, scale, causal != 0, nullptr,
                           nullptr, (hipStream_t)stream);
}

int fa_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
           const uint16_t* o, const uint16_t* dO, const float* lse,
           uint16_t* dq, uint16_t* dk, uint16_t* dv, void* workspace,
           size_t workspace_bytes, int B, int H, int N, int d, float scale,
           int causal, void* stream) {
  if (!q || !k || !v || !o || !dO || !lse || !dq || !dk || !dv)
    return FA_ERR_NULL;
  int st = check_shape_bwd(B, H, N, d);
  if (st != FA_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
      !aligned16(dO) || !aligned16(lse) || !aligned16(dq) || !aligned16(dk) ||
      !aligned16(dv))
    return FA_ERR_ALIGN;
  st = check_workspace(workspace, workspace_bytes, B, H, N);
  if (st != FA_OK) return st;
  st = fa_bwd_preprocess(o, dO, workspace, workspace_bytes, B, H, N, d, stream);
  if (st != FA_OK) return st;
  st = fa_bwd_dkdv(q, k, v, dO, lse, dk, dv, workspace, workspace_bytes, B, H,
                   N, d, scale, causal, stream);
  if (st != FA_OK) return st;
  return fa_bwd_dq(q, k, v, dO, lse, dq, workspace, workspace_bytes, B, H, N,
                   d, scale, causal, stream);
}

int fa_bwd_noalloc(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                   const uint16_t* o, const uint16_t* dO, const float* lse,
                   uint16_t* dq, uint16_t* dk, uint16_t* dv, int B, int H,
                   int N, int d, float scale, int causal, void* stream) {
  if (!q || !k || !v || !o || !dO || !lse || !dq || !dk || !dv)
    return FA_ERR_NULL;
  int st = check_shape_bwd(B, H, N, d);
  if (st != FA_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
      !aligned16(dO) || !aligned16(lse) || !aligned16(dq) || !aligned16(dk) ||
      !aligned16(dv))
    return FA_ERR_ALIGN;
  if ((long long)B * H * N > FA_BWD_NOALLOC_MAX_ROWS) return FA_ERR_TOO_LARGE;
  void* scratch = nullptr;
  if (fa::noalloc_scratch(&scratch) != 0) return FA_ERR_HIP;
  float* D = (float*)scratch;
  const hipStream_t s = (hipStream_t)stream;
  st = fa::launch_bwd_preprocess(o, dO, D, B, H, N, d, s);
  if (st != FA_OK) return st;
  st = fa::launch_bwd_dkdv(q, k, v, dO, lse, D, nullptr, dk, dv, B, H, N, d,
                           scale, causal != 0, nullptr, nullptr, s);
  if (st != FA_OK) return st;
  return fa::launch_bwd_dq(q, k, v, dO, lse, D, nullptr, dq, B, H, N, d,
                           scale, causal != 0, nullptr, nullptr, s);
}

int fa_bwd_kvlen(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                 const uint16_t* o, const uint16_t* dO, const float* lse,
                 const int32_t* kv_len, uint16_t* dq, uint16_t* dk,
                 uint16_t* dv, void* workspace, size_t workspace_bytes, int B,
                 int H, int N, int d, float scale, int causal, void* stream) {
  if (!q || !k || !v || !o || !dO || !lse || !dq || !dk || !dv)
    return FA_ERR_NULL;
  int st = check_shape_bwd(B, H, N, d);
  if (st != FA_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
      !aligned16(dO) || !aligned16(lse) || !aligned16(dq) || !aligned16(dk) ||
      !aligned16(dv) || ((uintptr_t)kv_len & 3u) != 0)
    return FA_ERR_ALIGN;
  st = check_workspace(workspace, workspace_bytes, B, H, N);
  if (st != FA_OK) return st;
  st = fa_bwd_preprocess(o, dO, workspace, workspace_bytes, B, H, N, d, stream);
  if (st != FA_OK) return st;
  st = fa::launch_bwd_dkdv(q, k, v, dO, lse, (const float*)workspace, nullptr,
                           dk, dv, B, H, N, d, scale, causal != 0, nullptr,
                           kv_len, (hipStream_t)stream);
  if (st != FA_OK) return FA_ERR_HIP;
  st = fa::launch_bwd_dq(q, k, v, dO, lse, (const float*)workspace, nullptr,
                         dq, B, H, N, d, scale, causal != 0, nullptr, kv_len,
                         (hipStream_t)stream);
  return st == 0 ? FA_OK : FA_ERR_HIP;
}

int fa_bwd_dkdv_block_sparse(const uint16_t* q, const uint16_t* k,
                             const uint16_t* v, const uint16_t* dO,
                             const float* lse, const uint8_t* block_mask,
                             uint16_t* dk, uint16_t* dv, const void* workspace,
                             size_t workspace_bytes, int B, int H, int N, int d,
                             float scale, int causal, void* stream) {
  if (!q || !k || !v || !dO || !lse || !block_mask || !dk || !dv)
    return FA_ERR_NULL;
  int st = check_shape_bwd(B, H, N, d);
  if (st != FA_OK) return st;
  if ((N + FA_SPARSE_BK - 1) / FA_SPARSE_BK > FA_SPARSE_MAX_KEY_BLOCKS)
    return FA_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dO) ||
      !aligned16(lse) || !aligned16(dk) || !aligned16(dv))
    return FA_ERR_ALIGN;
  st = check_workspace(workspace, workspace_bytes, B, H, N);
  if (st != FA_OK) return st;
  return fa::launch_bwd_dkdv(q, k, v, dO, lse, (const float*)workspace,
                             block_mask, dk, dv, B, H, N, d, scale,
                             causal != 0, nullptr, nullptr, (hipStream_t)stream);
}

int fa_bwd_dq_block_sparse(const uint16_t* q, const uint16_t* k,
                           const uint16_t* v, const uint16_t* dO,
                           const float* lse, const uint8_t* block_mask,
                           uint16_t* dq, const void* workspace,
                           size_t workspace_bytes, int B, int H, int N, int d,
                           float scale, int causal, void* stream) {
  if (!q || !k || !v || !dO || !lse || !block_mask || !dq) return FA_ERR_NULL;
  int st = check_shape_bwd(B, H, N, d);
  if (st != FA_OK) return st;
  if ((N + FA_SPARSE_BK - 1) / FA_SPARSE_BK > FA_SPARSE_MAX_KEY_BLOCKS)
    return FA_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dO) ||
      !aligned16(lse) || !aligned16(dq))
    return FA_ERR_ALIGN;
  st = check_workspace(workspace, workspace_bytes, B, H, N);
  if (st != FA_OK) return st;
  return fa::launch_bwd_dq(q, k, v, dO, lse, (const float*)workspace,
                           block_mask, dq, B, H, N, d, scale, causal != 0,
                           nullptr, nullptr, (hipStream_t)stream);
}

int fa_bwd_block_sparse(const uint16_t* q, const uint16_t* k,
                        const uint16_t* v, const uint16_t* o,
                        const uint16_t* dO, const float* lse,
                        const uint8_t* block_mask, uint16_t* dq, uint16_t* dk,
                        uint16_t* dv, void* workspace, size_t workspace_bytes,
                        int B, int H, int N, int d, float scale, int causal,
                        void* stream) {
  if (!q || !k || !v || !o || !dO || !lse || !block_mask || !dq || !dk || !dv)
    return FA_ERR_NULL;
  int st = check_shape_bwd(B, H, N, d);
  if (st != FA_OK) return st;
  if ((N + FA_SPARSE_BK - 1) / FA_SPARSE_BK > FA_SPARSE_MAX_KEY_BLOCKS)
    return FA_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
      !aligned16(dO) || !aligned16(lse) || !aligned16(dq) || !aligned16(dk) ||
      !aligned16(dv))
    return FA_ERR_ALIGN;
  st = check_workspace(workspace, workspace_bytes, B, H, N);
  if (st != FA_OK) return st;
  st = fa_bwd_preprocess(o, dO, workspace, workspace_bytes, B, H, N, d, stream);
  if (st != FA_OK) return st;
  st = fa_bwd_dkdv_block_sparse(q, k, v, dO, lse, block_mask, dk, dv,
                                workspace, workspace_bytes, B, H, N, d, scale,
                                causal, stream);
  if (st != FA_OK) return st;
  return fa_bwd_dq_block_sparse(q, k, v, dO, lse, block_mask, dq, workspace,
                                workspace_bytes, B, H, N, d, scale, causal,
                                stream);
}

int fa_fwd_dropout(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                   uint16_t* o, float* lse, int B, int H, int N, int d,
                   float scale, int causal, float p_drop, uint64_t seed,
                   uint32_t offset, void* stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  int st = check_shape(B, H, N, d);
  if (st != FA_OK) return st;
  fa::Dropout drop;
  st = make_dropout(p_drop, seed, offset, &drop);
  if (st != FA_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
      !aligned16(lse))
    return FA_ERR_ALIGN;
  return fa::launch_fwd_bf16(q, k, v, nullptr, nullptr, o, lse, B, H, N, d,
                             scale, causal != 0, &drop, (hipStream_t)stream);
}

int fa_bwd_dkdv_dropout(const uint16_t* q, const uint16_t* k,
                        const uint16_t* v, const uint16_t* dO,
                        const float* lse, uint16_t* dk, uint16_t* dv,
                        const void* workspace, size_t workspace_bytes, int B,
                        int H, int N, int d, float scale, int causal,
                        float p_drop, uint64_t seed, uint32_t offset,
                        void* stream) {
  if (!q || !k || !v || !dO || !lse || !dk || !dv) return FA_ERR_NULL;
  int st = check_shape_bwd(B, H, N, d);
  if (st != FA_OK) return st;
  fa::Dropout drop;
  st = make_dropout(p_drop, seed, offset, &drop);
  if (st != FA_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dO) ||
      !aligned16(lse) || !aligned16(dk) || !aligned16(dv))
    return FA_ERR_ALIGN;
  st = check_workspace(workspace, workspace_bytes, B, H, N);
  if (st != FA_OK) return st;
  return fa::launch_bwd_dkdv(q, k, v, dO, lse, (const float*)workspace,
                             nullptr, dk, dv, B, H, N, d, scale, causal != 0,
                             &drop, nullptr, (hipStream_t)stream);
}

int fa_bwd_dq_dropout(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                      const uint16_t* dO, const float* lse, uint16_t* dq,
                      const void* workspace, size_t workspace_bytes, int B,
                      int H, int N, int d, float scale, int causal,
                      float p_drop, uint64_t seed, uint32_t offset,
                      void* stream) {
  if (!q || !k || !v || !dO || !lse || !dq) return FA_ERR_NULL;
  int st = check_shape_bwd(B, H, N, d);
  if (st != FA_OK) return st;
  fa::Dropout drop;
  st = make_dropout(p_drop, seed, offset, &drop);
  if (st != FA_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dO) ||
      !aligned16(lse) || !aligned16(dq))
    return FA_ERR_ALIGN;
  st = check_workspace(workspace, workspace_bytes, B, H, N);
  if (st != FA_OK) return st;
  return fa::launch_bwd_dq(q, k, v, dO, lse, (const float*)workspace, nullptr,
                           dq, B, H, N, d, scale, causal != 0, &drop,
                           nullptr, (hipStream_t)stream);
}

int fa_bwd_dropout(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                   const uint16_t* o, const uint16_t* dO, const float* lse,
                   uint16_t* dq, uint16_t* dk, uint16_t* dv, void* workspace,
                   size_t workspace_bytes, int B, int H, int N, int d,
                   float scale, int causal, float p_drop, uint64_t seed,
                   uint32_t offset, void* stream) {
  if (!q || !k || !v || !o || !dO || !lse || !dq || !dk || !dv)
    return FA_ERR_NULL;
  int st = check_shape_bwd(B, H, N, d);
  if (st != FA_OK) return st;
  fa::Dropout drop;
  st = make_dropout(p_drop, seed, offset, &drop);
  if (st != FA_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
      !aligned16(dO) || !aligned16(lse) || !aligned16(dq) || !aligned16(dk) ||
      !aligned16(dv))
    return FA_ERR_ALIGN;
  st = check_workspace(workspace, workspace_bytes, B, H, N);
  if (st != FA_OK) return st;
  st = fa_bwd_preprocess(o, dO, workspace, workspace_bytes, B, H, N, d, stream);
  if (st != FA_OK) return st;
  st = fa_bwd_dkdv_dropout(q, k, v, dO, lse, dk, dv, workspace,
                           workspace_bytes, B, H, N, d, scale, causal, p_drop,
                           seed, offset, stream);
  if (st != FA_OK) return st;
  return fa_bwd_dq_dropout(q, k, v, dO, lse, dq, workspace, workspace_bytes,
                           B, H, N, d, scale, causal, p_drop, seed, offset,
                           stream);
}

}  // extern "C"
