// Internal launchers of libfa (not part of the C ABI).  Arguments are
// validated by the C-ABI layer before any of these is called; each returns 0
// or -6 (a HIP launch error).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

// Attention-dropout parameters (kernel argument).  Element (b, h, i, j)
// reads byte j % 4 of word i % 4 of Philox4x32-10 at counter
// (j / 4, i / 4, b H + h, offset) with key (k0, k1), and is kept iff that
// byte is >= p8.
struct Dropout {
  uint32_t k0, k1;    // key: the seed's low and high words
  uint32_t offset;    // fourth counter word
  int p8;             // byte threshold, 0..255
};

// kv_len: device int32 [B] or NULL; block_mask: device uint8
// [H, ceil(N/256), ceil(N/128)] or NULL; drop: dropout parameters or NULL
// (at most one of the three).
int launch_fwd_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                    const int32_t* kv_len, const uint8_t* block_mask,
                    uint16_t* o, float* lse, int B, int H, int N, int d,
                    float scale, int causal, const Dropout* drop,
                    hipStream_t stream);

int launch_fwd_f32(const float* q, const float* k, const float* v, float* o,
                   float* lse, int B, int H, int N, int d, float scale,
                   int causal, hipStream_t stream);

int launch_bwd_preprocess(const uint16_t* o, const uint16_t* dO, float* D,
                          int B, int H, int N, int d, hipStream_t stream);

// block_mask: device uint8 [H, ceil(N/256), ceil(N/128)] or NULL (dense);
// drop: dropout parameters or NULL (not both); kv_len: device int32 [B] key
// lengths or NULL (dense calls only).
int launch_bwd_dkdv(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                    const uint16_t* dO, const float* lse, const float* D,
                    const uint8_t* block_mask, uint16_t* dk, uint16_t* dv,
                    int B, int H, int N, int d, float scale, int causal,
                    const Dropout* drop, const int32_t* kv_len,
                    hipStream_t stream);

int launch_bwd_dq(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                  const uint16_t* dO, const float* lse, const float* D,
                  const uint8_t* block_mask, uint16_t* dq, int B, int H, int N,
                  int d, float scale, int causal, const Dropout* drop,
                  const int32_t* kv_len, hipStream_t stream);

// FP8 forward (layouts in include/fa.h).  signs: device int8 [d] or NULL.
int launch_fp8_quantize(const uint16_t* q, const uint16_t* k,
                        const uint16_t* v, const int8_t* signs, uint8_t* ws,
                        int B, int H, int N, int d, hipStream_t stream);

int launch_fwd_fp8(const uint8_t* ws, uint16_t* o, float* lse, int B, int H,
                   int N, int d, float score_scale, int causal,
                   hipStream_t stream);

// Compute units of the current device (hipDeviceAttributeMultiprocessorCount,
// read once per device; 256 if the query fails).
int device_cu_count();

// Device address of the fixed backward scratch (FA_BWD_NOALLOC_MAX_ROWS
// float32) on the current device, looked up once per device; 0 or -6.
int noalloc_scratch(void** addr);

// Causal linear attention forward (chunkwise).  ws: fp32 segment states
// of linear_workspace_bytes() bytes (NULL when that is 0).
size_t linear_workspace_bytes(int B, int H, int N, int d);
int launch_linear_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                      uint16_t* o, float* ws, int B, int H, int N, int d,
                      float scale, hipStream_t stream);
int launch_linear_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                      const uint16_t* dO, uint16_t* dq, uint16_t* dk,
                      uint16_t* dv, float* ws, int B, int H, int N, int d,
                      float scale, hipStream_t stream);

}  // namespace fa
