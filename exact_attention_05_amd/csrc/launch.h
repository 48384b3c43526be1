// Host-side launchers of the attention kernels.  Each returns the HIP error
// of its launch(es); shapes have been validated by the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace attn {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;  // may be null (not with merge)
  int B, H, N, d;
  float scale;
  int causal;
  bool merge = false;  // combine with the running (o, lse) instead of overwriting them
};

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t s);
hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t s);

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;  // may be null
  float* ws;   // U [BH][S][d], m [BH][S], l [BH][S]
  int B, H, L, d, splits;
  float scale;
};

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t s);

// Paged K/V cache: DecodeArgs.k/.v are the block pools, DecodeArgs.L unused.
struct PagedArgs {
  const int32_t* block_table;  // [B][max_blocks]
  const int32_t* seq_lens;     // [B]
  int max_blocks, num_blocks, log2_bs;
};

hipError_t launch_decode_paged_bf16(const DecodeArgs& a, const PagedArgs& p, hipStream_t s);

// The dense decode with its partials in a fixed per-device scratch of
// kDecodeScratchBytes (a.ws is ignored); the caller has checked that the
// partials fit.  Calls that overlap on one device share the scratch and race.
constexpr size_t kDecodeScratchBytes = size_t(32) << 20;
hipError_t launch_decode_noalloc_bf16(const DecodeArgs& a, hipStream_t s);

// FP8 forward: q, k, v are E4M3 [B, H, N, d]; fp32 scales per block of
// rows (32 for Q, 64 for K and V); o is bf16.
struct Fp8FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* q_scale;
  const float* k_scale;
  const float* v_scale;
  void* o;
  float* lse;  // may be null
  int B, H, N, d;
  float scale;
  int causal;
};

hipError_t launch_fwd_fp8(const Fp8FwdArgs& a, hipStream_t s);

// Block quantisation of a bf16 [B, H, N, d] tensor to E4M3 plus one fp32
// scale (max|x| / 448) per block of rows; signs (d values of +-1) turn on the
// Hadamard rotation.
struct QuantArgs {
  const void* x;
  const float* signs;  // may be null
  void* x8;
  float* scales;
  int B, H, N, d, block_rows;
};

hipError_t launch_quantize_fp8(const QuantArgs& a, hipStream_t s);

// Merge of two results over disjoint key sets; o/lse may alias o_a/lse_a or
// o_b/lse_b.
struct MergeArgs {
  const void* o_a;
  const float* lse_a;
  const void* o_b;
  const float* lse_b;
  void* o;
  float* lse;
  int B, H, N, d;
  bool bf16;
};

hipError_t launch_merge(const MergeArgs& a, hipStream_t s);

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dO;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* delta;  // workspace, 24 bytes per row: D [B*H*N] f32, -LSE*log2(e) [B*H*N] f32,
                 // three-part bf16 splits of -D and of -LSE/scale [B*H*N] x 8 bytes each
  int B, H, N, d;
  float scale;
  int causal;
  float* dqacc = nullptr;  // atomic-dQ variant: fp32 dQ accumulator [B*H*N*d]
};

hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t s);
hipError_t launch_bwd_atomic_bf16(const BwdArgs& a, hipStream_t s);

}  // namespace attn
