// Merge of two attention results over disjoint key sets: the partial-state
// merge of "FlashAttention 1 和 FlashAttention 2 的区别", section 6, for
// normalised outputs, which is the update each arriving K/V shard makes in
// Ring Attention ("FlashAttention", xuesongtap.github.io, section 5).  Per
// row: L = log(e^LSE_a + e^LSE_b), O = e^(LSE_a - L) O_a + e^(LSE_b - L) O_b.
//
// HBM-bound: each lane owns 8 consecutive values of one row (one 16-byte
// load of bf16, two of fp32), the D / 8 lanes of a row lie in one wavefront,
// so the row's LSE values are read before any lane writes them (in-place
// merges, O = O_a and LSE = LSE_a, are safe).
#include "common.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int kMergeThreads = 256;

template <typename T>
struct Vec8;
template <>
struct Vec8<__bf16> {
  __device__ static __forceinline__ void load(const __bf16* p, float (&x)[8]) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = bf16lo_to_f32(w[e]);
      x[2 * e + 1] = bf16hi_to_f32(w[e]);
    }
  }
  __device__ static __forceinline__ void store(__bf16* p, const float (&x)[8]) {
    const u32x4 w = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                     pack_bf16x2(x[6], x[7])};
    *reinterpret_cast<u32x4*>(p) = w;
  }
};
template <>
struct Vec8<float> {
  __device__ static __forceinline__ void load(const float* p, float (&x)[8]) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[e] = a[e];
      x[4 + e] = b[e];
    }
  }
  __device__ static __forceinline__ void store(float* p, const float (&x)[8]) {
    *reinterpret_cast<f32x4*>(p) = f32x4{x[0], x[1], x[2], x[3]};
    *reinterpret_cast<f32x4*>(p + 4) = f32x4{x[4], x[5], x[6], x[7]};
  }
};

template <int D, typename T>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(const T* Oa, const float* La, const T* Ob,
                                                              const float* Lb, T* O, float* L, int64_t rows) {
  constexpr int LPR = D / 8;  // lanes per row
  const int64_t row = (int64_t)blockIdx.x * (kMergeThreads / LPR) + threadIdx.x / LPR;
  const int u = threadIdx.x % LPR;
  if (row >= rows) return;
  const float la = La[row], lb = Lb[row];
  const float m = fmaxf(la, lb);
  const float base = (m == kNegInf) ? 0.f : m;
  const float wa = (la == kNegInf) ? 0.f : fast_exp2((la - base) * kLog2e);
  const float wb = (lb == kNegInf) ? 0.f : fast_exp2((lb - base) * kLog2e);
  const float tot = wa + wb;
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
  const float ca = wa * inv, cb = wb * inv;
  const int64_t off = row * D + 8 * u;
  float xa[8] = {}, xb[8] = {}, y[8];
  if (ca > 0.f) Vec8<T>::load(Oa + off, xa);  // an empty side's O is never read
  if (cb > 0.f) Vec8<T>::load(Ob + off, xb);
#pragma unroll
  for (int e = 0; e < 8; ++e) y[e] = ca * xa[e] + cb * xb[e];
  Vec8<T>::store(O + off, y);
  if (u == 0) L[row] = tot > 0.f ? base + fast_log2(tot) * kLn2 : kNegInf;
}

template <int D, typename T>
hipError_t run_merge(const MergeArgs& a, hipStream_t s) {
  const int64_t rows = (int64_t)a.B * a.H * a.N;
  constexpr int RPB = kMergeThreads / (D / 8);
  const int64_t grid = (rows + RPB - 1) / RPB;
  hipLaunchKernelGGL((merge_kernel<D, T>), dim3((unsigned)grid), dim3(kMergeThreads), 0, s,
                     static_cast<const T*>(a.o_a), a.lse_a, static_cast<const T*>(a.o_b), a.lse_b,
                     static_cast<T*>(a.o), a.lse, rows);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, hipStream_t s) {
  if (a.bf16) return a.d == 64 ? run_merge<64, __bf16>(a, s) : run_merge<128, __bf16>(a, s);
  return a.d == 64 ? run_merge<64, float>(a, s) : run_merge<128, float>(a, s);
}

}  // namespace attn
