// C ABI of libattn.so (declared in include/attn.h): argument validation on
// the host, then the kernel launchers.  No HIP call happens before every
// check has passed, so validation errors are testable without a GPU.
#include <math.h>
#include <stdint.h>

#include "attn.h"
#include "launch.h"

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool good_scale(float s) { return isfinite(s) && s > 0.f; }

// Validates the tensor pointers and the (B, H, N, d) sizes common to the
// forward and backward calls.
attn_status check_common(int B, int H, int N, int d, attn_dtype dtype, float scale) {
  if (B < 1 || H < 1 || N < 1 || d < 1) return ATTN_ERR_INVALID_ARG;
  if ((int64_t)B * H > INT32_MAX) return ATTN_ERR_INVALID_ARG;
  if (N > (1 << 24)) return ATTN_ERR_INVALID_ARG;
  if ((int64_t)B * H * (((int64_t)N + 63) / 64) > INT32_MAX) return ATTN_ERR_INVALID_ARG;
  if (!good_scale(scale)) return ATTN_ERR_INVALID_ARG;
  if (dtype != ATTN_F32 && dtype != ATTN_BF16) return ATTN_ERR_INVALID_ARG;
  return ATTN_OK;
}

bool tensor_ok(const void* p) { return p != nullptr && aligned(p, 16); }

attn_status from_hip(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP; }

}  // namespace

extern "C" {

const char* attn_status_string(attn_status s) {
  switch (s) {
    case ATTN_OK:
      return "ATTN_OK";
    case ATTN_ERR_INVALID_ARG:
      return "ATTN_ERR_INVALID_ARG: null or misaligned pointer, size out of range, or bad scale";
    case ATTN_ERR_UNSUPPORTED:
      return "ATTN_ERR_UNSUPPORTED: dtype/head_dim combination not built";
    case ATTN_ERR_WORKSPACE:
      return "ATTN_ERR_WORKSPACE: workspace missing or too small";
    case ATTN_ERR_HIP:
      return "ATTN_ERR_HIP: kernel launch failed";
    case ATTN_ERR_SCRATCH:
      return "ATTN_ERR_SCRATCH: the call needs more than the library's fixed scratch (ATTN_DECODE_SCRATCH_BYTES)";
  }
  return "unknown attn_status";
}

int attn_abi_version(void) { return 1; }

attn_status attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
                     attn_dtype dtype, float scale, int causal, void* stream) {
  attn_status st = check_common(B, H, N, d, dtype, scale);
  if (st != ATTN_OK) return st;
  if (!tensor_ok(q) || !tensor_ok(k) || !tensor_ok(v) || !tensor_ok(o)) return ATTN_ERR_INVALID_ARG;
  if (lse != nullptr && !aligned(lse, 4)) return ATTN_ERR_INVALID_ARG;
  const bool bf16_ok = dtype == ATTN_BF16 && (d == 64 || d == 128);
  const bool f32_ok = dtype == ATTN_F32 && d == 64;
  if (!bf16_ok && !f32_ok) return ATTN_ERR_UNSUPPORTED;
  attn::FwdArgs a{q, k, v, o, lse, B, H, N, d, scale, causal != 0};
  hipStream_t s = static_cast<hipStream_t>(stream);
  return from_hip(dtype == ATTN_BF16 ? attn::launch_fwd_bf16(a, s) : attn::launch_fwd_f32(a, s));
}

attn_status attn_fwd_merge(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
                           int d, attn_dtype dtype, float scale, int causal, void* stream) {
  attn_status st = check_common(B, H, N, d, dtype, scale);
  if (st != ATTN_OK) return st;
  if (!tensor_ok(q) || !tensor_ok(k) || !tensor_ok(v) || !tensor_ok(o)) return ATTN_ERR_INVALID_ARG;
  if (lse == nullptr || !aligned(lse, 4)) return ATTN_ERR_INVALID_ARG;
  if (!(dtype == ATTN_BF16 && (d == 64 || d == 128))) return ATTN_ERR_UNSUPPORTED;
  attn::FwdArgs a{q, k, v, o, lse, B, H, N, d, scale, causal != 0};
  a.merge = true;
  return from_hip(attn::launch_fwd_bf16(a, static_cast<hipStream_t>(stream)));
}

size_t attn_decode_workspace_bytes(int B, int H, int d, int num_splits) {
  if (B < 1 || H < 1 || d < 1 || num_splits < 1) return 0;
  return (size_t)B * (size_t)H * (size_t)num_splits * ((size_t)d + 2) * sizeof(float);
}

attn_status attn_fwd_splitk_decode(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                                   void* workspace, size_t workspace_bytes, int B, int H, int L, int d,
                                   int num_splits, attn_dtype dtype, float scale, void* stream) {
  if (B < 1 || H < 1 || L < 1 || L > (1 << 30) || d < 1) return ATTN_ERR_INVALID_ARG;
  if (num_splits < 1 || num_splits > 65535) return ATTN_ERR_INVALID_ARG;
  if ((int64_t)B * H * num_splits > INT32_MAX) return ATTN_ERR_INVALID_ARG;
  if (!good_scale(scale)) return ATTN_ERR_INVALID_ARG;
  if (dtype != ATTN_F32 && dtype != ATTN_BF16) return ATTN_ERR_INVALID_ARG;
  if (!tensor_ok(q) || !tensor_ok(k_cache) || !tensor_ok(v_cache) || !tensor_ok(o)) return ATTN_ERR_INVALID_ARG;
  if (lse != nullptr && !aligned(lse, 4)) return ATTN_ERR_INVALID_ARG;
  if (!(dtype == ATTN_BF16 && (d == 64 || d == 128))) return ATTN_ERR_UNSUPPORTED;
  if (workspace == nullptr || !aligned(workspace, 16)) return ATTN_ERR_WORKSPACE;
  if (workspace_bytes < attn_decode_workspace_bytes(B, H, d, num_splits)) return ATTN_ERR_WORKSPACE;
  attn::DecodeArgs a{q, k_cache, v_cache, o, lse, static_cast<float*>(workspace), B, H, L, d, num_splits, scale};
  return from_hip(attn::launch_decode_bf16(a, static_cast<hipStream_t>(stream)));
}

attn_status attn_fwd_splitk_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, void* o,
                                           float* lse, int B, int H, int L, int d, int num_splits, attn_dtype dtype,
                                           float scale, void* stream) {
  static_assert(ATTN_DECODE_SCRATCH_BYTES == attn::kDecodeScratchBytes, "scratch size");
  if (B < 1 || H < 1 || L < 1 || L > (1 << 30) || d < 1) return ATTN_ERR_INVALID_ARG;
  if (num_splits < 1 || num_splits > 65535) return ATTN_ERR_INVALID_ARG;
  if ((int64_t)B * H * num_splits > INT32_MAX) return ATTN_ERR_INVALID_ARG;
  if (!good_scale(scale)) return ATTN_ERR_INVALID_ARG;
  if (dtype != ATTN_F32 && dtype != ATTN_BF16) return ATTN_ERR_INVALID_ARG;
  if (!tensor_ok(q) || !tensor_ok(k_cache) || !tensor_ok(v_cache) || !tensor_ok(o)) return ATTN_ERR_INVALID_ARG;
  if (lse != nullptr && !aligned(lse, 4)) return ATTN_ERR_INVALID_ARG;
  if (!(dtype == ATTN_BF16 && (d == 64 || d == 128))) return ATTN_ERR_UNSUPPORTED;
  if (attn_decode_workspace_bytes(B, H, d, num_splits) > ATTN_DECODE_SCRATCH_BYTES) return ATTN_ERR_SCRATCH;
  attn::DecodeArgs a{q, k_cache, v_cache, o, lse, nullptr, B, H, L, d, num_splits, scale};
  return from_hip(attn::launch_decode_noalloc_bf16(a, static_cast<hipStream_t>(stream)));
}

attn_status attn_fwd_splitk_decode_paged(const void* q, const void* k_pool, const void* v_pool,
                                         const int* block_table, const int* seq_lens, void* o, float* lse,
                                         void* workspace, size_t workspace_bytes, int B, int H, int d,
                                         int num_blocks, int block_size, int max_blocks_per_seq, int num_splits,
                                         attn_dtype dtype, float scale, void* stream) {
  if (B < 1 || H < 1 || d < 1 || num_blocks < 1 || max_blocks_per_seq < 1) return ATTN_ERR_INVALID_ARG;
  if (block_size < 1 || (block_size & (block_size - 1)) != 0) return ATTN_ERR_INVALID_ARG;
  if ((int64_t)max_blocks_per_seq * block_size > (1 << 30)) return ATTN_ERR_INVALID_ARG;
  if (num_splits < 1 || num_splits > 65535) return ATTN_ERR_INVALID_ARG;
  if ((int64_t)B * H * num_splits > INT32_MAX) return ATTN_ERR_INVALID_ARG;
  if (!good_scale(scale)) return ATTN_ERR_INVALID_ARG;
  if (dtype != ATTN_F32 && dtype != ATTN_BF16) return ATTN_ERR_INVALID_ARG;
  if (!tensor_ok(q) || !tensor_ok(k_pool) || !tensor_ok(v_pool) || !tensor_ok(o)) return ATTN_ERR_INVALID_ARG;
  if (block_table == nullptr || !aligned(block_table, 4) || seq_lens == nullptr || !aligned(seq_lens, 4))
    return ATTN_ERR_INVALID_ARG;
  if (lse != nullptr && !aligned(lse, 4)) return ATTN_ERR_INVALID_ARG;
  if (!(dtype == ATTN_BF16 && (d == 64 || d == 128))) return ATTN_ERR_UNSUPPORTED;
  if (workspace == nullptr || !aligned(workspace, 16)) return ATTN_ERR_WORKSPACE;
  if (workspace_bytes < attn_decode_workspace_bytes(B, H, d, num_splits)) return ATTN_ERR_WORKSPACE;
  int log2_bs = 0;
  while ((1 << log2_bs) < block_size) ++log2_bs;
  attn::DecodeArgs a{q, k_pool, v_pool, o, lse, static_cast<float*>(workspace), B, H, 0, d, num_splits, scale};
  attn::PagedArgs p{block_table, seq_lens, max_blocks_per_seq, num_blocks, log2_bs};
  return from_hip(attn::launch_decode_paged_bf16(a, p, static_cast<hipStream_t>(stream)));
}

attn_status attn_quantize_fp8(const void* x, const float* signs, void* x8, float* scales, int B, int H, int N, int d,
                              int block_rows, void* stream) {
  if (B < 1 || H < 1 || N < 1 || N > (1 << 24) || d < 1 || block_rows < 1) return ATTN_ERR_INVALID_ARG;
  const int64_t nblk = ((int64_t)N + block_rows - 1) / block_rows;
  if ((int64_t)B * H * nblk > INT32_MAX) return ATTN_ERR_INVALID_ARG;
  if (!tensor_ok(x) || !tensor_ok(x8)) return ATTN_ERR_INVALID_ARG;
  if (scales == nullptr || !aligned(scales, 4)) return ATTN_ERR_INVALID_ARG;
  if (signs != nullptr && !aligned(signs, 4)) return ATTN_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  if (signs != nullptr && d != 64) return ATTN_ERR_UNSUPPORTED;
  attn::QuantArgs a{x, signs, x8, scales, B, H, N, d, block_rows};
  return from_hip(attn::launch_quantize_fp8(a, static_cast<hipStream_t>(stream)));
}

attn_status attn_fwd_fp8(const void* q8, const void* k8, const void* v8, const float* q_scale, const float* k_scale,
                         const float* v_scale, void* o, float* lse, int B, int H, int N, int d, int block_m,
                         int block_n, float scale, int causal, void* stream) {
  attn_status st = check_common(B, H, N, d, ATTN_BF16, scale);
  if (st != ATTN_OK) return st;
  if (block_m < 1 || block_n < 1) return ATTN_ERR_INVALID_ARG;
  if (!tensor_ok(q8) || !tensor_ok(k8) || !tensor_ok(v8) || !tensor_ok(o)) return ATTN_ERR_INVALID_ARG;
  for (const float* p : {q_scale, k_scale, v_scale})
    if (p == nullptr || !aligned(p, 4)) return ATTN_ERR_INVALID_ARG;
  if (lse != nullptr && !aligned(lse, 4)) return ATTN_ERR_INVALID_ARG;
  if (d != 64 || block_m != 32 || block_n != 64) return ATTN_ERR_UNSUPPORTED;
  attn::Fp8FwdArgs a{q8, k8, v8, q_scale, k_scale, v_scale, o, lse, B, H, N, d, scale, causal != 0};
  return from_hip(attn::launch_fwd_fp8(a, static_cast<hipStream_t>(stream)));
}

attn_status attn_merge(const void* o_a, const float* lse_a, const void* o_b, const float* lse_b, void* o, float* lse,
                       int B, int H, int N, int d, attn_dtype dtype, void* stream) {
  if (B < 1 || H < 1 || N < 1 || N > (1 << 24) || d < 1) return ATTN_ERR_INVALID_ARG;
  if ((int64_t)B * H * N > ((int64_t)1 << 40)) return ATTN_ERR_INVALID_ARG;
  if (dtype != ATTN_F32 && dtype != ATTN_BF16) return ATTN_ERR_INVALID_ARG;
  if (!tensor_ok(o_a) || !tensor_ok(o_b) || !tensor_ok(o)) return ATTN_ERR_INVALID_ARG;
  for (const float* p : {lse_a, lse_b, static_cast<const float*>(lse)})
    if (p == nullptr || !aligned(p, 4)) return ATTN_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  const int64_t rows = (int64_t)B * H * N;
  if ((rows + (256 / (d / 8)) - 1) / (256 / (d / 8)) > INT32_MAX) return ATTN_ERR_INVALID_ARG;
  attn::MergeArgs a{o_a, lse_a, o_b, lse_b, o, lse, B, H, N, d, dtype == ATTN_BF16};
  return from_hip(attn::launch_merge(a, static_cast<hipStream_t>(stream)));
}

size_t attn_bwd_workspace_bytes(int B, int H, int N) {
  if (B < 1 || H < 1 || N < 1) return 0;
  return (size_t)B * (size_t)H * (size_t)N * 24;
}

attn_status attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse,
                     void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, int B, int H, int N,
                     int d, attn_dtype dtype, float scale, int causal, void* stream) {
  attn_status st = check_common(B, H, N, d, dtype, scale);
  if (st != ATTN_OK) return st;
  if (!tensor_ok(q) || !tensor_ok(k) || !tensor_ok(v) || !tensor_ok(o) || !tensor_ok(dO) || !tensor_ok(dq) ||
      !tensor_ok(dk) || !tensor_ok(dv))
    return ATTN_ERR_INVALID_ARG;
  if (lse == nullptr || !aligned(lse, 4)) return ATTN_ERR_INVALID_ARG;
  if (!(dtype == ATTN_BF16 && (d == 64 || d == 128))) return ATTN_ERR_UNSUPPORTED;
  if (workspace == nullptr || !aligned(workspace, 16)) return ATTN_ERR_WORKSPACE;
  if (workspace_bytes < attn_bwd_workspace_bytes(B, H, N)) return ATTN_ERR_WORKSPACE;
  attn::BwdArgs a{q, k, v, o, dO, lse, dq, dk, dv, static_cast<float*>(workspace), B, H, N, d, scale, causal != 0};
  return from_hip(attn::launch_bwd_bf16(a, static_cast<hipStream_t>(stream)));
}

static size_t bwd_terms_bytes_aligned(int B, int H, int N) {
  return (attn_bwd_workspace_bytes(B, H, N) + 255) & ~(size_t)255;
}

size_t attn_bwd_atomic_workspace_bytes(int B, int H, int N, int d) {
  if (B < 1 || H < 1 || N < 1 || d < 1) return 0;
  return bwd_terms_bytes_aligned(B, H, N) + (size_t)B * (size_t)H * (size_t)N * (size_t)d * 4;
}

attn_status attn_bwd_atomic_dq(const void* q, const void* k, const void* v, const void* o, const void* dO,
                               const float* lse, void* dq, void* dk, void* dv, void* workspace,
                               size_t workspace_bytes, int B, int H, int N, int d, attn_dtype dtype,
                               float scale, int causal, void* stream) {
  attn_status st = check_common(B, H, N, d, dtype, scale);
  if (st != ATTN_OK) return st;
  if (!tensor_ok(q) || !tensor_ok(k) || !tensor_ok(v) || !tensor_ok(o) || !tensor_ok(dO) || !tensor_ok(dq) ||
      !tensor_ok(dk) || !tensor_ok(dv))
    return ATTN_ERR_INVALID_ARG;
  if (lse == nullptr || !aligned(lse, 4)) return ATTN_ERR_INVALID_ARG;
  if (!(dtype == ATTN_BF16 && (d == 64 || d == 128))) return ATTN_ERR_UNSUPPORTED;
  if (workspace == nullptr || !aligned(workspace, 16)) return ATTN_ERR_WORKSPACE;
  if (workspace_bytes < attn_bwd_atomic_workspace_bytes(B, H, N, d)) return ATTN_ERR_WORKSPACE;
  attn::BwdArgs a{q, k, v, o, dO, lse, dq, dk, dv, static_cast<float*>(workspace), B, H, N, d, scale, causal != 0};
  a.dqacc = reinterpret_cast<float*>(static_cast<unsigned char*>(workspace) + bwd_terms_bytes_aligned(B, H, N));
  return from_hip(attn::launch_bwd_atomic_bf16(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
