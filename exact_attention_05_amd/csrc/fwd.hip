// Exact attention forward, FA-2 loop order, for gfx950 (CDNA4).
//
// What is computed ("FlashAttention", xuesongtap.github.io, sections 1-3;
// "8. FlashAttention 实战", triton-tutorial.pages.dev, sections 8.3-8.4):
// for every query row i, O_i = sum_j softmax_j(scale * q_i . k_j) v_j and
// LSE_i = m_i + ln l_i, with the online state (m, l, U) carried across K/V
// tiles and O = U / l at the end.
//
// Mapping to the hardware:
//   * one workgroup = 4 wavefronts = a query tile of 4*32*QT rows; each
//     wavefront owns whole query rows (split-Q, "FlashAttention 1 和
//     FlashAttention 2 的区别", sections 7-8), so no cross-wave merge exists;
//   * Q stays in VGPRs as MFMA B operands for the whole K/V sweep;
//   * K/V tiles of 64 keys go HBM -> VGPR -> LDS, double-buffered: the loads
//     of tile j+1 are in flight while tile j is computed;
//   * the scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16, so each lane holds 32 scores of ONE query:
//     row max and row sum are in-lane plus one exchange with lane l^32;
//   * the exponentials are exp2 with log2(e) folded into the scale
//     (Triton tutorial, section 8.7.3); P~ is rounded to bf16 for the second
//     product (section 8.4.4) while l sums the fp32 values;
//   * O^T += V^T P~^T reuses the score accumulator directly as the B operand:
//     V is stored transposed in LDS with its 4-key chunks permuted to match
//     the accumulator's row order, so each lane reads 16 contiguous bytes;
//   * the causal mask is -inf on the diagonal tiles only; tiles above the
//     diagonal are never loaded, and wavefronts whose rows lie entirely above
//     a tile skip its arithmetic (Triton tutorial, section 8.7.1).
#include "common.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kBc = 64;  // keys per K/V tile
constexpr int kPad = 8;  // bf16 elements of LDS row padding (16 bytes)

template <int D>
struct FwdLds {
  static constexpr int kKRow = D + kPad;    // K tile: [64 keys][D], row stride
  static constexpr int kVRow = kBc + kPad;  // V^T tile: [D][64 keys], row stride
  static constexpr int kKElems = kBc * kKRow;
  static constexpr int kVElems = D * kVRow;
  static constexpr int kBufElems = kKElems + kVElems;
  static constexpr int kElems = 2 * kBufElems;
};

// Position of 4-key chunk kc inside the transposed V tile.  Within every
// 16-key group the accumulator supplies keys {0-3, 8-11} to lanes 0-31 and
// {4-7, 12-15} to lanes 32-63 of one MFMA; swapping the two low bits of the
// chunk index makes each of those sets 8 contiguous columns.
__device__ __forceinline__ int vt_chunk(int kc) { return (kc & ~3) | ((kc & 1) << 1) | ((kc >> 1) & 1); }

template <int D, int QT, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void fwd_bf16_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    __bf16* __restrict__ O, float* __restrict__ LSE, int N, int n_qtiles, int total_wg,
    float scale_log2) {
  using L = FwdLds<D>;
  constexpr int BR = kWaves * 32 * QT;
  constexpr int KCH = kBc * D / 8 / kThreads;   // 16-byte K chunks per thread
  constexpr int VBL = kBc * D / 16 / kThreads;  // 4x4 V blocks per thread
  __shared__ __attribute__((aligned(16))) __bf16 smem[L::kElems];

  const int lid = xcd_remap(blockIdx.x, total_wg);
  const int bh = lid / n_qtiles;
  int qtile = lid % n_qtiles;
  if (CAUSAL) qtile = n_qtiles - 1 - qtile;  // longest rows first

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int64_t base = (int64_t)bh * N * D;
  const __bf16* Qh = Q + base;
  const __bf16* Kh = K + base;
  const __bf16* Vh = V + base;
  __bf16* Oh = O + base;

  const int q0 = qtile * BR;
  const int qw0 = q0 + wave * 32 * QT;
  const int kend = CAUSAL ? min(N, q0 + BR) : N;
  const int nblk = (kend + kBc - 1) / kBc;

  // Q tile as MFMA B operands: lane holds Q[row][16ks + 8g .. +7].
  bf16x8 qf[QT][D / 16];
#pragma unroll
  for (int nt = 0; nt < QT; ++nt) {
    const int qr = qw0 + nt * 32 + l32;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      if (qr < N) {
        qf[nt][ks] = *reinterpret_cast<const bf16x8*>(Qh + (int64_t)qr * D + 16 * ks + 8 * g);
      } else {
        qf[nt][ks] = bf16x8{};
      }
    }
  }

  f32x16 oacc[QT][D / 32];
  float m2[QT], lsum[QT];
#pragma unroll
  for (int nt = 0; nt < QT; ++nt) {
    m2[nt] = kNegInf;
    lsum[nt] = 0.f;
#pragma unroll
    for (int mt = 0; mt < D / 32; ++mt) oacc[nt][mt] = f32x16{};
  }

  u32x4 kreg[KCH];
  u32x2 vreg[VBL][4];

  auto gload = [&](int kb) {
#pragma unroll
    for (int c = 0; c < KCH; ++c) {
      const int id = tid + c * kThreads;
      const int row = id / (D / 8), col = (id % (D / 8)) * 8;
      const int key = kb + row;
      kreg[c] = key < N ? *reinterpret_cast<const u32x4*>(Kh + (int64_t)key * D + col) : u32x4{};
    }
#pragma unroll
    for (int b = 0; b < VBL; ++b) {
      const int id = tid + b * kThreads;
      const int kc = id / (D / 4), dc = id % (D / 4);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = kb + 4 * kc + r;
        vreg[b][r] = key < N ? *reinterpret_cast<const u32x2*>(Vh + (int64_t)key * D + 4 * dc) : u32x2{};
      }
    }
  };

  auto sstore = [&](int buf) {
    __bf16* Ks = smem + buf * L::kBufElems;
    __bf16* Vt = Ks + L::kKElems;
#pragma unroll
    for (int c = 0; c < KCH; ++c) {
      const int id = tid + c * kThreads;
      const int row = id / (D / 8), col = (id % (D / 8)) * 8;
      *reinterpret_cast<u32x4*>(Ks + row * L::kKRow + col) = kreg[c];
    }
#pragma unroll
    for (int b = 0; b < VBL; ++b) {
      const int id = tid + b * kThreads;
      const int kc = id / (D / 4), dc = id % (D / 4);
      const int pcol = 4 * vt_chunk(kc);
      // 4 keys x 4 dims -> 4 dims x 4 keys (bf16 pairs)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int w = i >> 1;
        const bool hi = i & 1;
        uint32_t e[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) e[r] = hi ? (vreg[b][r][w] >> 16) : (vreg[b][r][w] & 0xffffu);
        u32x2 out = {e[0] | (e[1] << 16), e[2] | (e[3] << 16)};
        *reinterpret_cast<u32x2*>(Vt + (4 * dc + i) * L::kVRow + pcol) = out;
      }
    }
  };

  if (nblk > 0) {
    gload(0);
    sstore(0);
  }
  __syncthreads();

  for (int j = 0; j < nblk; ++j) {
    const int kb = j * kBc;
    const int buf = j & 1;
    if (j + 1 < nblk) gload(kb + kBc);
    const __bf16* Ks = smem + buf * L::kBufElems;
    const __bf16* Vt = Ks + L::kKElems;

    const bool active = !CAUSAL || kb <= qw0 + 32 * QT - 1;
    if (active) {
      // S^T = K_j Q^T: [64 keys] x [32 queries] per (kh, nt)
      f32x16 sacc[QT][2];
#pragma unroll
      for (int nt = 0; nt < QT; ++nt) sacc[nt][0] = sacc[nt][1] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(Ks + (32 * kh + l32) * L::kKRow + 16 * ks + 8 * g);
#pragma unroll
          for (int nt = 0; nt < QT; ++nt) sacc[nt][kh] = mfma32x32x16(a, qf[nt][ks], sacc[nt][kh]);
        }
      }

      const bool need_mask = (kb + kBc > N) || (CAUSAL && kb + kBc - 1 > qw0);
      if (need_mask) {
#pragma unroll
        for (int nt = 0; nt < QT; ++nt) {
          const int qr = qw0 + nt * 32 + l32;
#pragma unroll
          for (int kh = 0; kh < 2; ++kh) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int key = kb + 32 * kh + acc_row(i, g);
              const bool vis = key < N && (!CAUSAL || key <= qr);
              if (!vis) sacc[nt][kh][i] = kNegInf;
            }
          }
        }
      }

      bf16x8 pb[QT][4];
#pragma unroll
      for (int nt = 0; nt < QT; ++nt) {
        float mx = kNegInf;
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[nt][kh][i]);
        mx = fmaxf(mx, shfl_xor_f32(mx, 32));
        const float mnew = fmaxf(m2[nt], mx * scale_log2);
        const float msafe = (mnew == kNegInf) ? 0.f : mnew;
        const float alpha = fast_exp2(m2[nt] - msafe);
        m2[nt] = mnew;
        float rs = 0.f;
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float p = fast_exp2(fmaf(sacc[nt][kh][i], scale_log2, -msafe));
            sacc[nt][kh][i] = p;
            rs += p;
          }
        lsum[nt] = lsum[nt] * alpha + rs;
#pragma unroll
        for (int mt = 0; mt < D / 32; ++mt) oacc[nt][mt] *= alpha;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          float x[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = sacc[nt][t >> 1][8 * (t & 1) + e];
          pb[nt][t] = pack_bf16x8(x);
        }
      }

      // O^T += V_j^T P~^T
#pragma unroll
      for (int t = 0; t < 4; ++t) {
#pragma unroll
        for (int mt = 0; mt < D / 32; ++mt) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(Vt + (32 * mt + l32) * L::kVRow + 16 * t + 8 * g);
#pragma unroll
          for (int nt = 0; nt < QT; ++nt) oacc[nt][mt] = mfma32x32x16(a, pb[nt][t], oacc[nt][mt]);
        }
      }
    }

    if (j + 1 < nblk) sstore(buf ^ 1);
    __syncthreads();
  }

  // Epilogue: O = U / l (bf16, RNE) and LSE = (m2 + log2 l) * ln 2.
#pragma unroll
  for (int nt = 0; nt < QT; ++nt) {
    const int qr = qw0 + nt * 32 + l32;
    const float lt = lsum[nt] + shfl_xor_f32(lsum[nt], 32);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    if (qr < N) {
#pragma unroll
      for (int mt = 0; mt < D / 32; ++mt) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int d0 = 32 * mt + 8 * c + 4 * g;
          u32x2 w = {pack_bf16x2(oacc[nt][mt][4 * c] * inv, oacc[nt][mt][4 * c + 1] * inv),
                     pack_bf16x2(oacc[nt][mt][4 * c + 2] * inv, oacc[nt][mt][4 * c + 3] * inv)};
          *reinterpret_cast<u32x2*>(Oh + (int64_t)qr * D + d0) = w;
        }
      }
      if (g == 0 && LSE != nullptr)
        LSE[(int64_t)bh * N + qr] = lt > 0.f ? (m2[nt] + fast_log2(lt)) * kLn2 : kNegInf;
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 inputs, d = 64: same loop with v_mfma_f32_32x32x2_f32; P~ stays fp32
// and V needs no transpose (one fp32 per lane per MFMA operand).
// ---------------------------------------------------------------------------
constexpr int kF32D = 64;
constexpr int kF32Row = kF32D + 4;

template <bool CAUSAL>
__global__ __launch_bounds__(kThreads) void fwd_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ O, float* __restrict__ LSE, int N, int n_qtiles, int total_wg, float scale_log2) {
  constexpr int D = kF32D;
  constexpr int BR = kWaves * 32;
  constexpr int KCH = kBc * D / 4 / kThreads;  // 16-byte chunks per thread (K and V each)
  constexpr int kBuf = 2 * kBc * kF32Row;      // K then V, fp32
  __shared__ __attribute__((aligned(16))) float smem[2 * kBuf];

  const int lid = xcd_remap(blockIdx.x, total_wg);
  const int bh = lid / n_qtiles;
  int qtile = lid % n_qtiles;
  if (CAUSAL) qtile = n_qtiles - 1 - qtile;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int64_t base = (int64_t)bh * N * D;
  const float* Qh = Q + base;
  const float* Kh = K + base;
  const float* Vh = V + base;
  float* Oh = O + base;

  const int q0 = qtile * BR;
  const int qw0 = q0 + wave * 32;
  const int qr = qw0 + l32;
  const int kend = CAUSAL ? min(N, q0 + BR) : N;
  const int nblk = (kend + kBc - 1) / kBc;

  float qf[D / 2];  // lane holds Q[qr][2ks + g]
#pragma unroll
  for (int ks = 0; ks < D / 2; ++ks) qf[ks] = qr < N ? Qh[(int64_t)qr * D + 2 * ks + g] : 0.f;

  f32x16 oacc[D / 32];
#pragma unroll
  for (int mt = 0; mt < D / 32; ++mt) oacc[mt] = f32x16{};
  float m2 = kNegInf, lsum = 0.f;

  f32x4 kreg[KCH], vreg[KCH];
  auto gload = [&](int kb) {
#pragma unroll
    for (int c = 0; c < KCH; ++c) {
      const int id = tid + c * kThreads;
      const int row = id / (D / 4), col = (id % (D / 4)) * 4;
      const int key = kb + row;
      kreg[c] = key < N ? *reinterpret_cast<const f32x4*>(Kh + (int64_t)key * D + col) : f32x4{};
      vreg[c] = key < N ? *reinterpret_cast<const f32x4*>(Vh + (int64_t)key * D + col) : f32x4{};
    }
  };
  auto sstore = [&](int buf) {
    float* Ks = smem + buf * kBuf;
    float* Vs = Ks + kBc * kF32Row;
#pragma unroll
    for (int c = 0; c < KCH; ++c) {
      const int id = tid + c * kThreads;
      const int row = id / (D / 4), col = (id % (D / 4)) * 4;
      *reinterpret_cast<f32x4*>(Ks + row * kF32Row + col) = kreg[c];
      *reinterpret_cast<f32x4*>(Vs + row * kF32Row + col) = vreg[c];
    }
  };

  if (nblk > 0) {
    gload(0);
    sstore(0);
  }
  __syncthreads();

  for (int j = 0; j < nblk; ++j) {
    const int kb = j * kBc;
    const int buf = j & 1;
    if (j + 1 < nblk) gload(kb + kBc);
    const float* Ks = smem + buf * kBuf;
    const float* Vs = Ks + kBc * kF32Row;
    const bool active = !CAUSAL || kb <= qw0 + 31;
    if (active) {
      f32x16 sacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int ks = 0; ks < D / 2; ++ks)
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
          sacc[kh] = mfma32x32x2f32(Ks[(32 * kh + l32) * kF32Row + 2 * ks + g], qf[ks], sacc[kh]);

      const bool need_mask = (kb + kBc > N) || (CAUSAL && kb + kBc - 1 > qw0);
      if (need_mask) {
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = kb + 32 * kh + acc_row(i, g);
            if (!(key < N && (!CAUSAL || key <= qr))) sacc[kh][i] = kNegInf;
          }
      }
      float mx = kNegInf;
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kh][i]);
      mx = fmaxf(mx, shfl_xor_f32(mx, 32));
      const float mnew = fmaxf(m2, mx * scale_log2);
      const float msafe = (mnew == kNegInf) ? 0.f : mnew;
      const float alpha = fast_exp2(m2 - msafe);
      m2 = mnew;
      float rs = 0.f;
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = fast_exp2(fmaf(sacc[kh][i], scale_log2, -msafe));
          sacc[kh][i] = p;
          rs += p;
        }
      lsum = lsum * alpha + rs;
#pragma unroll
      for (int mt = 0; mt < D / 32; ++mt) oacc[mt] *= alpha;
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = 32 * kh + acc_row(i, g);
#pragma unroll
          for (int mt = 0; mt < D / 32; ++mt)
            oacc[mt] = mfma32x32x2f32(Vs[key * kF32Row + 32 * mt + l32], sacc[kh][i], oacc[mt]);
        }
    }
    if (j + 1 < nblk) sstore(buf ^ 1);
    __syncthreads();
  }

  const float lt = lsum + shfl_xor_f32(lsum, 32);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (qr < N) {
#pragma unroll
    for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int d0 = 32 * mt + 8 * c + 4 * g;
        f32x4 w = {oacc[mt][4 * c] * inv, oacc[mt][4 * c + 1] * inv, oacc[mt][4 * c + 2] * inv,
                   oacc[mt][4 * c + 3] * inv};
        *reinterpret_cast<f32x4*>(Oh + (int64_t)qr * D + d0) = w;
      }
    if (g == 0 && LSE != nullptr) LSE[(int64_t)bh * N + qr] = lt > 0.f ? (m2 + fast_log2(lt)) * kLn2 : kNegInf;
  }
}

template <int D, int QT, bool CAUSAL>
hipError_t run_bf16(const FwdArgs& a, hipStream_t s) {
  constexpr int BR = kWaves * 32 * QT;
  const int n_qtiles = (a.N + BR - 1) / BR;
  const int total = n_qtiles * a.B * a.H;
  const float scale_log2 = a.scale * kLog2e;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, QT, CAUSAL>), dim3(total), dim3(kThreads), 0, s,
                     static_cast<const __bf16*>(a.q), static_cast<const __bf16*>(a.k),
                     static_cast<const __bf16*>(a.v), static_cast<__bf16*>(a.o), a.lse, a.N, n_qtiles,
                     total, scale_log2);
  return hipGetLastError();
}

template <bool CAUSAL>
hipError_t run_f32(const FwdArgs& a, hipStream_t s) {
  constexpr int BR = kWaves * 32;
  const int n_qtiles = (a.N + BR - 1) / BR;
  const int total = n_qtiles * a.B * a.H;
  hipLaunchKernelGGL((fwd_f32_kernel<CAUSAL>), dim3(total), dim3(kThreads), 0, s,
                     static_cast<const float*>(a.q), static_cast<const float*>(a.k),
                     static_cast<const float*>(a.v), static_cast<float*>(a.o), a.lse, a.N, n_qtiles, total,
                     a.scale * kLog2e);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t s) {
  if (a.d == 64) return a.causal ? run_bf16<64, 1, true>(a, s) : run_bf16<64, 1, false>(a, s);
  return a.causal ? run_bf16<128, 1, true>(a, s) : run_bf16<128, 1, false>(a, s);
}

hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t s) {
  return a.causal ? run_f32<true>(a, s) : run_f32<false>(a, s);
}

}  // namespace attn
