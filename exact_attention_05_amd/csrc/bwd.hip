// Exact attention backward by recomputation for gfx950 ("8. FlashAttention
// 实战", triton-tutorial.pages.dev, section 8.8; "FlashAttention",
// xuesongtap.github.io, section 3).
//
// Three launches on one stream, no atomics, bitwise deterministic:
//   bwd_preprocess : D_i = sum_d dO_id O_id (fp32), from the saved O.
//   bwd_dkdv       : key tiles outer.  Each wavefront owns 32 keys, keeps
//                    K, V in VGPRs and dK^T, dV^T as fp32 MFMA accumulators,
//                    and streams 64-row query tiles (Q, dO, LSE, D) through
//                    LDS:  S = Q K^T, P = exp(S - LSE), dP = dO V^T,
//                    dS = P o (dP - D), dV^T += dO^T P, dK^T += Q^T dS.
//   bwd_dq         : query tiles outer.  Each wavefront owns 32 queries,
//                    keeps Q, dO in VGPRs and dQ^T as accumulator, and
//                    streams 64-key tiles (K, K^T, V) through LDS:
//                    S^T = K Q^T, dP^T = V dO^T, dS^T = P^T o (dP^T - D),
//                    dQ^T += K^T dS^T.
// dK and dQ are multiplied by the softmax scale at the end (section 8.8.4).
// Products whose contraction runs over the sequence take their P / dS
// operand straight from the accumulator of the previous product, and their
// other operand from a transposed LDS copy whose 4-row chunks are permuted
// to the accumulator's row order (the same scheme as V^T in the forward).
#include "common.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kPad = 8;
constexpr int kT = 64;  // rows per streamed tile

__device__ __forceinline__ int vt_chunk(int kc) { return (kc & ~3) | ((kc & 1) << 1) | ((kc >> 1) & 1); }

// A 64 x D bf16 tile held by the workgroup as 4x4 blocks (4 rows x 8 bytes).
template <int D>
struct Blocks4 {
  static constexpr int NB = kT * D / 16 / kThreads;
  u32x2 r[NB][4];

  __device__ __forceinline__ void load(const __bf16* src, int rows_valid, int tid) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int id = tid + b * kThreads;
      const int kc = id / (D / 4), dc = id % (D / 4);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int row = 4 * kc + rr;
        r[b][rr] = row < rows_valid ? *reinterpret_cast<const u32x2*>(src + (int64_t)row * D + 4 * dc) : u32x2{};
      }
    }
  }
  __device__ __forceinline__ void store_rows(__bf16* dst, int stride, int tid) const {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int id = tid + b * kThreads;
      const int kc = id / (D / 4), dc = id % (D / 4);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) *reinterpret_cast<u32x2*>(dst + (4 * kc + rr) * stride + 4 * dc) = r[b][rr];
    }
  }
  // dst is [D][stride]; row chunk kc lands at column 4 * vt_chunk(kc).
  __device__ __forceinline__ void store_transposed(__bf16* dst, int stride, int tid) const {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int id = tid + b * kThreads;
      const int kc = id / (D / 4), dc = id % (D / 4);
      const int pcol = 4 * vt_chunk(kc);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int w = i >> 1;
        const bool hi = i & 1;
        uint32_t e[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) e[rr] = hi ? (r[b][rr][w] >> 16) : (r[b][rr][w] & 0xffffu);
        u32x2 out = {e[0] | (e[1] << 16), e[2] | (e[3] << 16)};
        *reinterpret_cast<u32x2*>(dst + (4 * dc + i) * stride + pcol) = out;
      }
    }
  }
};

// A 64 x D bf16 tile held as 16-byte row chunks.
template <int D>
struct Chunks16 {
  static constexpr int NC = kT * D / 8 / kThreads;
  u32x4 r[NC];
  __device__ __forceinline__ void load(const __bf16* src, int rows_valid, int tid) {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int id = tid + c * kThreads;
      const int row = id / (D / 8), col = (id % (D / 8)) * 8;
      r[c] = row < rows_valid ? *reinterpret_cast<const u32x4*>(src + (int64_t)row * D + col) : u32x4{};
    }
  }
  __device__ __forceinline__ void store_rows(__bf16* dst, int stride, int tid) const {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int id = tid + c * kThreads;
      const int row = id / (D / 8), col = (id % (D / 8)) * 8;
      *reinterpret_cast<u32x4*>(dst + row * stride + col) = r[c];
    }
  }
};

// Store a D^T x 32 accumulator tile set (lane: column l32, rows acc_row) as
// rows of a [rows][D] bf16 tensor, multiplied by `mul`.
template <int D>
__device__ __forceinline__ void store_transposed_acc(__bf16* dst_row, const f32x16 (&acc)[D / 32], int g,
                                                     float mul) {
#pragma unroll
  for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int d0 = 32 * mt + 8 * c + 4 * g;
      u32x2 w = {pack_bf16x2(acc[mt][4 * c] * mul, acc[mt][4 * c + 1] * mul),
                 pack_bf16x2(acc[mt][4 * c + 2] * mul, acc[mt][4 * c + 3] * mul)};
      *reinterpret_cast<u32x2*>(dst_row + d0) = w;
    }
}

// ---------------------------------------------------------------------------
// D = rowsum(dO o O)
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_preprocess_kernel(const __bf16* __restrict__ O,
                                                                  const __bf16* __restrict__ dO,
                                                                  float* __restrict__ delta, int64_t rows) {
  constexpr int LPR = D / 8;  // lanes per row
  const int64_t row = (int64_t)blockIdx.x * (kThreads / LPR) + threadIdx.x / LPR;
  const int u = threadIdx.x % LPR;
  float acc = 0.f;
  if (row < rows) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(O + row * D + 8 * u);
    const u32x4 b = *reinterpret_cast<const u32x4*>(dO + row * D + 8 * u);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      acc = fmaf(bf16lo_to_f32(a[w]), bf16lo_to_f32(b[w]), acc);
      acc = fmaf(bf16hi_to_f32(a[w]), bf16hi_to_f32(b[w]), acc);
    }
  }
#pragma unroll
  for (int m = 1; m < LPR; m <<= 1) acc += shfl_xor_f32(acc, m);
  if (row < rows && u == 0) delta[row] = acc;
}

// ---------------------------------------------------------------------------
// dK, dV: key tiles outer
// ---------------------------------------------------------------------------
template <int D>
struct DkdvLds {
  static constexpr int kRow = D + kPad;   // Q, dO row-major [64][D]
  static constexpr int kTRow = kT + kPad; // Q^T, dO^T [D][64]
  static constexpr int kRowElems = kT * kRow;
  static constexpr int kTElems = D * kTRow;
  static constexpr int kBufBf16 = 2 * kRowElems + 2 * kTElems;
  static constexpr int kBufBytes = kBufBf16 * 2 + 2 * kT * 4;  // + LSE2, D
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void bwd_dkdv_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const __bf16* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ delta,
    __bf16* __restrict__ dK, __bf16* __restrict__ dV, int N, int n_ktiles, int total_wg, float scale,
    float scale_log2) {
  using Lds = DkdvLds<D>;
  constexpr int BK = kWaves * 32;
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * Lds::kBufBytes];

  const int lid = xcd_remap(blockIdx.x, total_wg);
  const int bh = lid / n_ktiles;
  const int ktile = lid % n_ktiles;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int64_t base = (int64_t)bh * N * D;
  const int k0 = ktile * BK;
  const int kw0 = k0 + wave * 32;
  const int key = kw0 + l32;

  // K, V of this wavefront's 32 keys as B operands: lane holds row `key`, dims 16ks + 8g .. +7
  bf16x8 kB[D / 16], vB[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    if (key < N) {
      kB[ks] = *reinterpret_cast<const bf16x8*>(K + base + (int64_t)key * D + 16 * ks + 8 * g);
      vB[ks] = *reinterpret_cast<const bf16x8*>(V + base + (int64_t)key * D + 16 * ks + 8 * g);
    } else {
      kB[ks] = bf16x8{};
      vB[ks] = bf16x8{};
    }
  }
  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int mt = 0; mt < D / 32; ++mt) dk[mt] = dv[mt] = f32x16{};

  const int i_begin = CAUSAL ? k0 / kT : 0;
  const int i_end = (N + kT - 1) / kT;

  Blocks4<D> qreg, doreg;
  float lse_r = 0.f, del_r = 0.f;

  auto gload = [&](int it) {
    const int q0 = it * kT;
    const int rows = min(kT, N - q0);
    qreg.load(Q + base + (int64_t)q0 * D, rows, tid);
    doreg.load(dO + base + (int64_t)q0 * D, rows, tid);
    if (tid < kT) {
      const int qi = q0 + tid;
      lse_r = qi < N ? LSE[(int64_t)bh * N + qi] * kLog2e : __builtin_inff();
      del_r = qi < N ? delta[(int64_t)bh * N + qi] : 0.f;
    }
  };
  auto sstore = [&](int buf) {
    __bf16* Qs = reinterpret_cast<__bf16*>(smem + buf * Lds::kBufBytes);
    __bf16* dOs = Qs + Lds::kRowElems;
    __bf16* Qt = dOs + Lds::kRowElems;
    __bf16* dOt = Qt + Lds::kTElems;
    float* ls = reinterpret_cast<float*>(dOt + Lds::kTElems);
    qreg.store_rows(Qs, Lds::kRow, tid);
    qreg.store_transposed(Qt, Lds::kTRow, tid);
    doreg.store_rows(dOs, Lds::kRow, tid);
    doreg.store_transposed(dOt, Lds::kTRow, tid);
    if (tid < kT) {
      ls[tid] = lse_r;
      ls[kT + tid] = del_r;
    }
  };

  if (i_begin < i_end) {
    gload(i_begin);
    sstore(0);
  }
  __syncthreads();

  for (int it = i_begin; it < i_end; ++it) {
    const int buf = (it - i_begin) & 1;
    const int q0 = it * kT;
    if (it + 1 < i_end) gload(it + 1);
    const __bf16* Qs = reinterpret_cast<const __bf16*>(smem + buf * Lds::kBufBytes);
    const __bf16* dOs = Qs + Lds::kRowElems;
    const __bf16* Qt = dOs + Lds::kRowElems;
    const __bf16* dOt = Qt + Lds::kTElems;
    const float* ls = reinterpret_cast<const float*>(dOt + Lds::kTElems);

    const bool active = !CAUSAL || q0 + kT - 1 >= kw0;
    if (active) {
      f32x16 sacc[2], dpacc[2];
      sacc[0] = sacc[1] = dpacc[0] = dpacc[1] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
#pragma unroll
        for (int qh = 0; qh < 2; ++qh) {
          const bf16x8 aq = *reinterpret_cast<const bf16x8*>(Qs + (32 * qh + l32) * Lds::kRow + 16 * ks + 8 * g);
          const bf16x8 ad = *reinterpret_cast<const bf16x8*>(dOs + (32 * qh + l32) * Lds::kRow + 16 * ks + 8 * g);
          sacc[qh] = mfma32x32x16(aq, kB[ks], sacc[qh]);
          dpacc[qh] = mfma32x32x16(ad, vB[ks], dpacc[qh]);
        }
      }
      const bool need_mask = CAUSAL && q0 < kw0 + 31;
      // P = exp2(S*c - LSE2), dS = P o (dP - D); lane holds queries q0 + 32qh + acc_row(i, g)
#pragma unroll
      for (int qh = 0; qh < 2; ++qh) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int qo = 32 * qh + 8 * c + 4 * g;
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(ls + qo);
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(ls + kT + qo);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = 4 * c + r;
            float p = fast_exp2(fmaf(sacc[qh][i], scale_log2, -l4[r]));
            if (need_mask && key > q0 + qo + r) p = 0.f;
            sacc[qh][i] = p;
            dpacc[qh][i] = p * (dpacc[qh][i] - d4[r]);
          }
        }
      }
      bf16x8 pb[4], sb[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        float x[8], y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          x[e] = sacc[t >> 1][8 * (t & 1) + e];
          y[e] = dpacc[t >> 1][8 * (t & 1) + e];
        }
        pb[t] = pack_bf16x8(x);
        sb[t] = pack_bf16x8(y);
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
#pragma unroll
        for (int mt = 0; mt < D / 32; ++mt) {
          const bf16x8 ado = *reinterpret_cast<const bf16x8*>(dOt + (32 * mt + l32) * Lds::kTRow + 16 * t + 8 * g);
          const bf16x8 aq = *reinterpret_cast<const bf16x8*>(Qt + (32 * mt + l32) * Lds::kTRow + 16 * t + 8 * g);
          dv[mt] = mfma32x32x16(ado, pb[t], dv[mt]);
          dk[mt] = mfma32x32x16(aq, sb[t], dk[mt]);
        }
      }
    }
    if (it + 1 < i_end) sstore(buf ^ 1);
    __syncthreads();
  }

  if (key < N) {
    store_transposed_acc<D>(dV + base + (int64_t)key * D, dv, g, 1.f);
    store_transposed_acc<D>(dK + base + (int64_t)key * D, dk, g, scale);
  }
}

// ---------------------------------------------------------------------------
// dQ: query tiles outer
// ---------------------------------------------------------------------------
template <int D>
struct DqLds {
  static constexpr int kRow = D + kPad;   // K, V row-major [64][D]
  static constexpr int kTRow = kT + kPad; // K^T [D][64]
  static constexpr int kRowElems = kT * kRow;
  static constexpr int kTElems = D * kTRow;
  static constexpr int kBufElems = 2 * kRowElems + kTElems;
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void bwd_dq_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                                                          const __bf16* __restrict__ V,
                                                          const __bf16* __restrict__ dO,
                                                          const float* __restrict__ LSE,
                                                          const float* __restrict__ delta, __bf16* __restrict__ dQ,
                                                          int N, int n_qtiles, int total_wg, float scale,
                                                          float scale_log2) {
  using Lds = DqLds<D>;
  constexpr int BQ = kWaves * 32;
  __shared__ __attribute__((aligned(16))) __bf16 smem[2 * Lds::kBufElems];

  const int lid = xcd_remap(blockIdx.x, total_wg);
  const int bh = lid / n_qtiles;
  int qtile = lid % n_qtiles;
  if (CAUSAL) qtile = n_qtiles - 1 - qtile;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int64_t base = (int64_t)bh * N * D;
  const int q0 = qtile * BQ;
  const int qw0 = q0 + wave * 32;
  const int qr = qw0 + l32;

  bf16x8 qB[D / 16], doB[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    if (qr < N) {
      qB[ks] = *reinterpret_cast<const bf16x8*>(Q + base + (int64_t)qr * D + 16 * ks + 8 * g);
      doB[ks] = *reinterpret_cast<const bf16x8*>(dO + base + (int64_t)qr * D + 16 * ks + 8 * g);
    } else {
      qB[ks] = bf16x8{};
      doB[ks] = bf16x8{};
    }
  }
  const float lse2 = qr < N ? LSE[(int64_t)bh * N + qr] * kLog2e : __builtin_inff();
  const float dl = qr < N ? delta[(int64_t)bh * N + qr] : 0.f;

  f32x16 dq[D / 32];
#pragma unroll
  for (int mt = 0; mt < D / 32; ++mt) dq[mt] = f32x16{};

  const int kend = CAUSAL ? min(N, q0 + BQ) : N;
  const int nblk = (kend + kT - 1) / kT;

  Blocks4<D> kreg;
  Chunks16<D> vreg;
  auto gload = [&](int j) {
    const int kb = j * kT;
    const int rows = min(kT, N - kb);
    kreg.load(K + base + (int64_t)kb * D, rows, tid);
    vreg.load(V + base + (int64_t)kb * D, rows, tid);
  };
  auto sstore = [&](int buf) {
    __bf16* Ks = smem + buf * Lds::kBufElems;
    __bf16* Vs = Ks + Lds::kRowElems;
    __bf16* Kt = Vs + Lds::kRowElems;
    kreg.store_rows(Ks, Lds::kRow, tid);
    kreg.store_transposed(Kt, Lds::kTRow, tid);
    vreg.store_rows(Vs, Lds::kRow, tid);
  };

  if (nblk > 0) {
    gload(0);
    sstore(0);
  }
  __syncthreads();

  for (int j = 0; j < nblk; ++j) {
    const int kb = j * kT;
    const int buf = j & 1;
    if (j + 1 < nblk) gload(j + 1);
    const __bf16* Ks = smem + buf * Lds::kBufElems;
    const __bf16* Vs = Ks + Lds::kRowElems;
    const __bf16* Kt = Vs + Lds::kRowElems;
    const bool active = !CAUSAL || kb <= qw0 + 31;
    if (active) {
      f32x16 sacc[2], dpacc[2];
      sacc[0] = sacc[1] = dpacc[0] = dpacc[1] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
          const bf16x8 ak = *reinterpret_cast<const bf16x8*>(Ks + (32 * kh + l32) * Lds::kRow + 16 * ks + 8 * g);
          const bf16x8 av = *reinterpret_cast<const bf16x8*>(Vs + (32 * kh + l32) * Lds::kRow + 16 * ks + 8 * g);
          sacc[kh] = mfma32x32x16(ak, qB[ks], sacc[kh]);
          dpacc[kh] = mfma32x32x16(av, doB[ks], dpacc[kh]);
        }
      }
      const bool need_mask = (kb + kT > N) || (CAUSAL && kb + kT - 1 > qw0);
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float p = fast_exp2(fmaf(sacc[kh][i], scale_log2, -lse2));
          if (need_mask) {
            const int kk = kb + 32 * kh + acc_row(i, g);
            if (kk >= N || (CAUSAL && kk > qr)) p = 0.f;
          }
          dpacc[kh][i] = p * (dpacc[kh][i] - dl);
        }
      }
      bf16x8 sb[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        float y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = dpacc[t >> 1][8 * (t & 1) + e];
        sb[t] = pack_bf16x8(y);
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
#pragma unroll
        for (int mt = 0; mt < D / 32; ++mt) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(Kt + (32 * mt + l32) * Lds::kTRow + 16 * t + 8 * g);
          dq[mt] = mfma32x32x16(a, sb[t], dq[mt]);
        }
      }
    }
    if (j + 1 < nblk) sstore(buf ^ 1);
    __syncthreads();
  }

  if (qr < N) store_transposed_acc<D>(dQ + base + (int64_t)qr * D, dq, g, scale);
}

template <int D, bool CAUSAL>
hipError_t run_bwd(const BwdArgs& a, hipStream_t s) {
  const int BH = a.B * a.H;
  const int64_t rows = (int64_t)BH * a.N;
  constexpr int rows_per_wg = kThreads / (D / 8);
  hipLaunchKernelGGL((bwd_preprocess_kernel<D>), dim3((unsigned)((rows + rows_per_wg - 1) / rows_per_wg)),
                     dim3(kThreads), 0, s, static_cast<const __bf16*>(a.o), static_cast<const __bf16*>(a.dO),
                     a.delta, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  const float scale_log2 = a.scale * kLog2e;
  const int n_kt = (a.N + kWaves * 32 - 1) / (kWaves * 32);
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), dim3(n_kt * BH), dim3(kThreads), 0, s,
                     static_cast<const __bf16*>(a.q), static_cast<const __bf16*>(a.k),
                     static_cast<const __bf16*>(a.v), static_cast<const __bf16*>(a.dO), a.lse, a.delta,
                     static_cast<__bf16*>(a.dk), static_cast<__bf16*>(a.dv), a.N, n_kt, n_kt * BH, a.scale,
                     scale_log2);
  e = hipGetLastError();
  if (e != hipSuccess) return e;

  const int n_qt = (a.N + kWaves * 32 - 1) / (kWaves * 32);
  hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL>), dim3(n_qt * BH), dim3(kThreads), 0, s,
                     static_cast<const __bf16*>(a.q), static_cast<const __bf16*>(a.k),
                     static_cast<const __bf16*>(a.v), static_cast<const __bf16*>(a.dO), a.lse, a.delta,
                     static_cast<__bf16*>(a.dq), a.N, n_qt, n_qt * BH, a.scale, scale_log2);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t s) {
  if (a.d == 64) return a.causal ? run_bwd<64, true>(a, s) : run_bwd<64, false>(a, s);
  return a.causal ? run_bwd<128, true>(a, s) : run_bwd<128, false>(a, s);
}

}  // namespace attn
