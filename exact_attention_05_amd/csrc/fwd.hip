// Exact attention forward, FA-2 loop order, for gfx950 (CDNA4).
//
// What is computed ("FlashAttention", xuesongtap.github.io, sections 1-3;
// "8. FlashAttention 实战", triton-tutorial.pages.dev, sections 8.3-8.4):
// for every query row i, O_i = sum_j softmax_j(scale * q_i . k_j) v_j and
// LSE_i = m_i + ln l_i, with the online state (m, l, U) carried across K/V
// tiles and O = U / l at the end.
//
// Mapping to the hardware:
//   * every wavefront owns 32 whole query rows (split-Q, "FlashAttention 1 和
//     FlashAttention 2 的区别", sections 7-8), so no cross-wave merge exists;
//     d = 128: 4 wavefronts per workgroup (fwd_bf16_kernel); d = 64: 8
//     wavefronts in two groups one phase apart, two workgroups per CU (four
//     wavefronts per SIMD), so matrix and vector work of different
//     wavefronts overlap (fwd_pp4_kernel);
//   * Q stays in VGPRs as MFMA B operands for the whole K/V sweep;
//   * K/V tiles of 64 keys go HBM -> LDS with direct-to-LDS copies into a
//     ring of buffers in the swizzled tile layout of common.h, copied ahead
//     of their use;
//   * the scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16, so each lane holds 32 scores of ONE query:
//     row max and row sum are in-lane plus one exchange with lane l^32;
//   * the exponentials are exp2 with log2(e) folded into the scale
//     (Triton tutorial, section 8.7.3); P~ is rounded to bf16 for the second
//     product (section 8.4.4) while l sums the fp32 values;
//   * O^T += V^T P~^T takes P~ straight from the score accumulator as the B
//     operand; V^T comes from the row-major V tile through transposing LDS
//     reads (ds_read_b64_tr_b16) whose 4-key chunks follow the accumulator's
//     row order;
//   * the causal mask is -inf on the diagonal tiles only; tiles above the
//     diagonal are never loaded, and the longest query tiles are dispatched
//     first (Triton tutorial, section 8.7.1).  d = 64: a wavefront stops
//     computing after its last key tile with a visible key, and the two
//     wavefronts of a SIMD own row blocks s and 7 - s of the query tile, so
//     every SIMD has the same share of the diagonal.
//   * attn_fwd_merge instantiates the same kernels with MERGE: the epilogue
//     reads the row's running (O, LSE) and writes the result over both key
//     sets (see merge_weights), so a Ring Attention step is one launch.
#include "common.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kBc = 64;  // keys per K/V tile

// Reference point of the exponentials.  The online state (m, l, U) is exact
// for ANY reference m as long as l, U and the LSE all use the same one
// (O = U / l and LSE = m + ln l cancel it), and numerically m only has to keep
// every P~ = 2^(s*c - m) finite.  So m is set to the exact row max on the
// first K/V tile and afterwards moves only when a lane's partial row sum of a
// tile exceeds kSumLimit (or overflows): then the tile's exponentials are
// redone with the exact running max, U and l rescaled, as in the plain online
// update.  For ordinary inputs that never happens after the first tile, which
// removes the per-tile row max and the rescale of U from the inner loop.
// With partial sums below 2^64, U stays below 2^64 * N * max|v|.
constexpr float kSumLimit = 18446744073709551616.f;  // 2^64

// Fused merge (attn_fwd_merge): the result over the keys of earlier calls,
// (O_prev, LSE_prev) in memory, and over this call's keys, (U / l, LSE_new),
// combine into the result over both sets: with L = log(e^LSE_prev +
// e^LSE_new), O = e^(LSE_prev - L) O_prev + e^(LSE_new - L) U / l ("Ring
// Attention", the online-softmax update across key blocks).  Base 2 inside;
// a side with LSE = -inf gets weight 0 and its O is not used.
struct MergeWeights {
  float wa, wb;  // weights of O_prev and of U / l, summing to 1 (both 0 if both sides are empty)
  float lse;     // L
};
__device__ __forceinline__ MergeWeights merge_weights(float lse_prev, float lse2_new) {
  const float a2 = lse_prev * kLog2e;
  const float mx = fmaxf(a2, lse2_new);
  if (mx == kNegInf) return {0.f, 0.f, kNegInf};
  const float wa = fast_exp2(a2 - mx), wb = fast_exp2(lse2_new - mx);
  const float tot = wa + wb;
  const float r = 1.f / tot;
  return {wa * r, wb * r, (mx + fast_log2(tot)) * kLn2};
}
// O of one lane's 4 consecutive dims: the new values x, merged with the bf16
// values at dst when MERGE (dst is read before it is written, by this lane only)
template <bool MERGE>
__device__ __forceinline__ u32x2 merged_out4(const __bf16* dst, float x0, float x1, float x2, float x3,
                                             const MergeWeights& w) {
  if constexpr (MERGE) {
    const u32x2 prev = *reinterpret_cast<const u32x2*>(dst);
    float p[4] = {bf16lo_to_f32(prev[0]), bf16hi_to_f32(prev[0]), bf16lo_to_f32(prev[1]), bf16hi_to_f32(prev[1])};
    const bool use_prev = w.wa > 0.f;
    x0 = (use_prev ? w.wa * p[0] : 0.f) + w.wb * x0;
    x1 = (use_prev ? w.wa * p[1] : 0.f) + w.wb * x1;
    x2 = (use_prev ? w.wa * p[2] : 0.f) + w.wb * x2;
    x3 = (use_prev ? w.wa * p[3] : 0.f) + w.wb * x3;
  }
  return u32x2{pack_bf16x2(x0, x1), pack_bf16x2(x2, x3)};
}

template <int D, int QT, int NBUF, bool CAUSAL, bool MERGE = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void fwd_bf16_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    __bf16* __restrict__ O, float* __restrict__ LSE, int N, int n_qtiles, int total_wg,
    float scale_log2) {
  using T = TileLayout<D>;
  constexpr int BR = kWaves * 32 * QT;
  constexpr int NLD = D / 32;  // direct-to-LDS copies per wavefront per tile and tensor
  // A ring of NBUF buffers, each a K tile then a V tile; tile j uses buffer
  // j % NBUF and is copied NBUF - 1 tiles ahead of its use.  Each buffer is
  // its own LDS object and the tile loop is unrolled by NBUF, so the compiler
  // can tell reads of one buffer from copies still landing in another (it
  // would otherwise wait for every copy before the first LDS read).
  static_assert(NBUF >= 2 && NBUF <= 4, "ring depth");
  __shared__ __attribute__((aligned(1024))) unsigned char sb0[2 * T::kBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char sb1[2 * T::kBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char sb2[NBUF > 2 ? 2 * T::kBytes : 16];
  __shared__ __attribute__((aligned(1024))) unsigned char sb3[NBUF > 3 ? 2 * T::kBytes : 16];
  auto ring = [&](int b) -> unsigned char* { return b == 0 ? sb0 : b == 1 ? sb1 : b == 2 ? sb2 : sb3; };

  const int lid = xcd_remap(blockIdx.x, total_wg);
  const int bh = lid / n_qtiles;
  int qtile = lid % n_qtiles;
  if (CAUSAL) qtile = n_qtiles - 1 - qtile;  // longest rows first

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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

  // Copy geometry: copy i of this wavefront fills lines 4*(wave*NLD + i) ..
  // +3 of a tile; lane l fills physical chunk l%16 of line +l/16, i.e. the
  // logical (key, chunk) that the swizzle maps there.
  int ld_key[NLD], ld_col[NLD];
#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    const int line = 4 * (wave * NLD + i) + (lane >> 4);
    int k, c;
    T::at(line, lane & 15, k, c);
    ld_key[i] = k;
    ld_col[i] = 8 * c;
  }
  auto issue_tile_copy = [&](int kb, int buf) {
    unsigned char* kt = ring(buf);
    unsigned char* vt = kt + T::kBytes;
    // one buffer descriptor per tile: keys past N read zeros (masked out)
    const uint32_t bytes = (uint32_t)(N - kb) * (uint32_t)(D * 2);
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int voff = (ld_key[i] * D + ld_col[i]) * 2;
      const int lds_line = 4 * (wave * NLD + i);
      buffer_to_lds16(Kh + (int64_t)kb * D, bytes, voff, kt + lds_line * 256);
      buffer_to_lds16(Vh + (int64_t)kb * D, bytes, voff, vt + lds_line * 256);
    }
  };

  // Per-lane LDS read offsets.
  // K operand of S^T = K Q^T: key 32kh + l32, chunk 2ks + g.
  int koff[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) koff[ks] = T::offset(l32, 2 * ks + g);
  constexpr int kKhStep = 32 * D * 2;  // 32 keys further: same swizzle phase
  // V^T operand of O^T += V^T P~^T through transposing reads: source lane
  // s = lane%16 of group G = lane/16 names key 16t + 8h + 4(G/2) + s/4 and
  // dims 32mt + 16(G%2) + 4(s%4) .. +3.
  int voff[2][D / 32];
  {
    const int s = lane & 15, G = lane >> 4;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int mt = 0; mt < D / 32; ++mt) {
        const int key = 8 * h + 4 * (G >> 1) + (s >> 2);
        const int dim = 32 * mt + 16 * (G & 1) + 4 * (s & 3);
        voff[h][mt] = T::offset(key, dim >> 3) + 8 * ((dim >> 2) & 1);
      }
  }
  constexpr int kTStep = 16 * D * 2;  // 16 keys further: same swizzle phase

  // Raw scores S^T of the current tile: sacc[nt][kh] holds keys 32kh..+31
  // against query rows qw0 + 32nt + l32.
  f32x16 sacc[QT][2];

  // S^T for key half kh of the tile at kt, all query tiles (K reads shared).
  auto scores_half = [&](const unsigned char* kt, int kh) {
#pragma unroll
    for (int nt = 0; nt < QT; ++nt) sacc[nt][kh] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(kt + koff[ks] + kh * kKhStep);
#pragma unroll
      for (int nt = 0; nt < QT; ++nt) sacc[nt][kh] = mfma32x32x16(a, qf[nt][ks], sacc[nt][kh]);
    }
  };

  auto mask_half = [&](int kb, int kh) {
#pragma unroll
    for (int nt = 0; nt < QT; ++nt) {
      const int qr = qw0 + nt * 32 + l32;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kb + 32 * kh + acc_row(i, g);
        const bool vis = key < N && (!CAUSAL || key <= qr);
        if (!vis) sacc[nt][kh][i] = kNegInf;
      }
    }
  };

  // P~ = 2^(s*c - m) for key half kh of query tile nt, rounded to bf16
  // straight into the B operands pb[nt][2kh], pb[nt][2kh+1] of the second
  // product (raw scores stay in sacc); rs[nt] gets the lane's fp32 partial
  // sum.  Returns true when that sum is too large or m is not set yet.
  float rs[QT];
  bf16x8 pb[QT][4];
  auto exponentials = [&](int nt, int kh) {
    const float msafe = (m2[nt] == kNegInf) ? 0.f : m2[nt];
    float r2[2];
#pragma unroll
    for (int th = 0; th < 2; ++th) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = fast_exp2(fmaf(sacc[nt][kh][8 * th + e], scale_log2, -msafe));
      r2[th] = ((x[0] + x[1]) + (x[2] + x[3])) + ((x[4] + x[5]) + (x[6] + x[7]));
      pb[nt][2 * kh + th] = pack_bf16x8(x);
    }
    rs[nt] = r2[0] + r2[1];
    return !(rs[nt] <= kSumLimit) || m2[nt] == kNegInf;
  };

  // Slow path for key half kh of query tile nt: move m up to the exact
  // running max (over the scores seen so far), rescale U and l by
  // alpha = 2^(m_old - m_new) (0 while m_old = -inf), redo the exponentials.
  auto rescue = [&](int nt, int kh) {
    float t4[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      t4[e] = fmaxf(fmaxf(sacc[nt][kh][4 * e], sacc[nt][kh][4 * e + 1]),
                    fmaxf(sacc[nt][kh][4 * e + 2], sacc[nt][kh][4 * e + 3]));
    float mx = fmaxf(fmaxf(t4[0], t4[1]), fmaxf(t4[2], t4[3]));
    mx = fmaxf(mx, shfl_xor_f32(mx, 32));
    const float mx2 = mx * scale_log2;
    const bool grow = mx2 > m2[nt];
    const float alpha = grow ? fast_exp2(m2[nt] - mx2) : 1.f;
    m2[nt] = grow ? mx2 : m2[nt];
    lsum[nt] *= alpha;
#pragma unroll
    for (int mt = 0; mt < D / 32; ++mt) oacc[nt][mt] *= alpha;
    exponentials(nt, kh);
  };

  // O^T += V^T P~^T for the 32 keys of half kh (V reads shared by the query tiles).
  auto pv_half = [&](const unsigned char* vt, int kh) {
#pragma unroll
    for (int th = 0; th < 2; ++th) {
      const int t = 2 * kh + th;
#pragma unroll
      for (int mt = 0; mt < D / 32; ++mt) {
        const u32x2 lo = lds_read_tr16(vt + voff[0][mt] + t * kTStep);
        const u32x2 hi = lds_read_tr16(vt + voff[1][mt] + t * kTStep);
        const u32x4 w = {lo[0], lo[1], hi[0], hi[1]};
        const bf16x8 a = bitcast<bf16x8>(w);
#pragma unroll
        for (int nt = 0; nt < QT; ++nt) oacc[nt][mt] = mfma32x32x16(a, pb[nt][t], oacc[nt][mt]);
      }
    }
  };

  // Instruction interleave for a step that overlaps MFMAs with the
  // exponentials of the other key half: per MFMA, its LDS operand reads and
  // an equal share of the vector ALU work.
  constexpr int kStepMfma = (D / 16) * QT;          // = 2 * (D / 32) * QT
  constexpr int kValuPerMfma = (56 * QT) / kStepMfma;

  // One wave-uniform branch for all query tiles, so that every exponential
  // of the step is needed before it (and stays in the step's block).
  auto check_half = [&](int kh) {
    bool bad = false;
#pragma unroll
    for (int nt = 0; nt < QT; ++nt) bad |= !(rs[nt] <= kSumLimit) || m2[nt] == kNegInf;
    if (__ballot(bad)) {
#pragma unroll
      for (int nt = 0; nt < QT; ++nt)
        if (__ballot(!(rs[nt] <= kSumLimit) || m2[nt] == kNegInf)) rescue(nt, kh);
    }
#pragma unroll
    for (int nt = 0; nt < QT; ++nt) lsum[nt] += rs[nt];
  };

#pragma unroll
  for (int p = 0; p < NBUF - 1; ++p)
    if (p < nblk) issue_tile_copy(p * kBc, p);

  for (int j0 = 0; j0 < nblk; j0 += NBUF) {
#pragma unroll
  for (int u = 0; u < NBUF; ++u) {
    const int j = j0 + u;
    if (j >= nblk) break;
    const int kb = j * kBc;
    // Tile j's copies are done when at most the copies of the NBUF - 2
    // tiles after it are still in flight (2 * NLD per tile and wavefront);
    // the barrier then makes every wavefront's part visible and guarantees
    // that nobody still reads the buffer the next copy overwrites.
    if (j + NBUF - 2 < nblk) {
      wait_vm_at_most<(NBUF - 2) * 2 * NLD>();
    } else {
      wait_vm_at_most<0>();
    }
    lds_barrier();
    if (j + NBUF - 1 < nblk) issue_tile_copy(kb + (NBUF - 1) * kBc, (u + NBUF - 1) % NBUF);
    const unsigned char* kt = ring(u);
    const unsigned char* vt = kt + T::kBytes;

    const bool active = !CAUSAL || kb <= qw0 + 32 * QT - 1;
    if (active) {
      const bool need_mask = (kb + kBc > N) || (CAUSAL && kb + kBc - 1 > qw0);
      // step 0: scores of key half 0
      scores_half(kt, 0);
      if (need_mask) mask_half(kb, 0);
      // step 1: scores of key half 1 | exponentials of key half 0
      scores_half(kt, 1);
#pragma unroll
      for (int nt = 0; nt < QT; ++nt) exponentials(nt, 0);
#pragma unroll
      for (int i = 0; i < kStepMfma; ++i) {
        if (i < D / 16) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, kValuPerMfma, 0);
      }
      check_half(0);
      if (need_mask) mask_half(kb, 1);
      // step 2: P~V of key half 0 | exponentials of key half 1
      pv_half(vt, 0);
#pragma unroll
      for (int nt = 0; nt < QT; ++nt) exponentials(nt, 1);
#pragma unroll
      for (int i = 0; i < kStepMfma; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x100, (D / 8) / kStepMfma > 0 ? (D / 8) / kStepMfma : 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, kValuPerMfma, 0);
      }
      check_half(1);
      // step 3: P~V of key half 1
      pv_half(vt, 1);
    }
  }
  }

  // Epilogue: O = U / l (bf16, RNE) and LSE = (m + log2 l) * ln 2, or
  // with MERGE both combined with the running result in O and LSE.
#pragma unroll
  for (int nt = 0; nt < QT; ++nt) {
    const int qr = qw0 + nt * 32 + l32;
    const float lt = lsum[nt] + shfl_xor_f32(lsum[nt], 32);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const float lse2 = lt > 0.f ? m2[nt] + fast_log2(lt) : kNegInf;
    if (qr < N) {
      MergeWeights mw{0.f, 1.f, lse2 * kLn2};
      if constexpr (MERGE) mw = merge_weights(LSE[(int64_t)bh * N + qr], lse2);
#pragma unroll
      for (int mt = 0; mt < D / 32; ++mt) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int d0 = 32 * mt + 8 * c + 4 * g;
          __bf16* dst = Oh + (int64_t)qr * D + d0;
          *reinterpret_cast<u32x2*>(dst) =
              merged_out4<MERGE>(dst, oacc[nt][mt][4 * c] * inv, oacc[nt][mt][4 * c + 1] * inv,
                                 oacc[nt][mt][4 * c + 2] * inv, oacc[nt][mt][4 * c + 3] * inv, mw);
        }
      }
      if (g == 0 && LSE != nullptr) LSE[(int64_t)bh * N + qr] = mw.lse;
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
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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

// ---------------------------------------------------------------------------
// d = 64 forward, four wavefronts per SIMD.  Eight wavefronts of 32 query
// rows (256 rows per workgroup); wavefronts 0-3 lead and 4-7 trail by one
// phase, so on every SIMD one wavefront of the workgroup is in a matrix phase
// while the other is in a vector phase, and two workgroups share each CU (80
// KB of LDS each), drifting freely against each other.  A single wavefront
// can issue only a fraction of what a SIMD executes -- about three quarters of
// the MFMA rate and half of the VALU rate -- so four per SIMD keep both units
// busier; with two workgroups each barrier holds 8 wavefronts, not 16, and
// the shorter query tiles balance causal grids better.  Per 64-key tile j:
// M(j) = O^T += V_{j-1}^T P~_{j-1}^T, then S_j^T = K_j Q^T (operands read from
// LDS in the phase); V(j) = mask, exponentials, bf16 P~, row sums.
//
// Ring of 5 tile buffers (K | V): tile j+3 is copied at M(j) into the slot of
// tile j-2, whose last reader (the trail's M(j-1)) is one phase earlier; each
// wavefront copies 1 KB of the K tile and 1 KB of the V tile.
// Each wavefront waits for its own copies of tile j+1 before the barrier that
// opens its V(j); for the trail that barrier opens the lead's M(j+1), the
// first reader of tile j+1.  Online state and reference rule as in
// fwd_bf16_kernel.
// ---------------------------------------------------------------------------
template <bool CAUSAL, bool MERGE = false>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4, 4))) void fwd_pp4_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    __bf16* __restrict__ O, float* __restrict__ LSE, int N, int n_qtiles, int total_wg, float scale_log2) {
  constexpr int D = 64;
  using T = TileLayout<D>;
  constexpr int NW = 8;
  constexpr int BR = NW * 32;
  __shared__ __attribute__((aligned(1024))) unsigned char sb0[2 * T::kBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char sb1[2 * T::kBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char sb2[2 * T::kBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char sb3[2 * T::kBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char sb4[2 * T::kBytes];

  int bh, qtile;
  causal_order<CAUSAL>(blockIdx.x, total_wg, n_qtiles, bh, qtile);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool lead = wave < NW / 2;
  const int g = lane >> 5, l32 = lane & 31;
  const int64_t base = (int64_t)bh * N * D;
  const int q0 = qtile * BR;
  // the lead and the trail wavefront of SIMD s (w = s and w = s + 4) own row
  // blocks s and 7 - s, so on a causal diagonal every SIMD has the same work
  const int qw0 = q0 + 32 * (wave < 4 ? wave : 11 - wave);
  const int qr = qw0 + l32;
  const int kend = CAUSAL ? min(N, q0 + BR) : N;
  const int ntiles = (kend + kBc - 1) / kBc;

  // each wavefront copies one 1 KB piece of the K tile and one of the V tile
  // (two direct-to-LDS buffer loads per tile; keys past N read zeros)
  const TileCopyBuf<D, NW> cp(wave, lane);
  auto issue_tile = [&](int j, unsigned char* buf) __attribute__((always_inline)) {
    cp.issue(K + base, N, j * kBc, buf);
    cp.issue(V + base, N, j * kBc, buf + T::kBytes);
  };

  // Q first: loads complete in issue order, so the first step waits for Q
  // and tile 0 only
  bf16x8 qB[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks)
    qB[ks] = qr < N ? *reinterpret_cast<const bf16x8*>(Q + base + (int64_t)qr * D + 16 * ks + 8 * g) : bf16x8{};
  issue_tile(0, sb0);

  const TileOffsets<D> of(lane);
  f32x16 oacc[D / 32];
#pragma unroll
  for (int mt = 0; mt < D / 32; ++mt) oacc[mt] = f32x16{};
  float m2 = kNegInf, lsum = 0.f, rs = 0.f;
  f32x16 sacc[2];  // S^T of the current tile, two halves of 32 keys
  bf16x8 pb[4];    // P~ of the current tile, four 16-key operands

  // S^T = K Q^T for the tile whose K is at kt.
  auto scores = [&](const unsigned char* kt) __attribute__((always_inline)) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      sacc[hh] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) sacc[hh] = mfma32x32x16(of.row(kt, ks, hh), qB[ks], sacc[hh]);
    }
  };
  // M: O^T += V^T P~^T of the previous tile (at bprev), then S^T of this one (at kt).
  auto mph = [&](const unsigned char* kt, const unsigned char* bprev, const bool do_pv, const bool do_s)
      __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(1);
    if (do_pv) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int mt = 0; mt < D / 32; ++mt) oacc[mt] = mfma32x32x16(of.tr(bprev + T::kBytes, t, mt), pb[t], oacc[mt]);
    }
    if (do_s) scores(kt);
    __builtin_amdgcn_s_setprio(0);
  };

  auto mask_tile = [&](int j) __attribute__((always_inline)) {
    const int kb = j * kBc;
    if ((kb + kBc > N) || (CAUSAL && kb + kBc - 1 > qw0)) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kb + 32 * hh + acc_row(i, g);
          const bool vis = key < N && (!CAUSAL || key <= qr);
          if (!vis) sacc[hh][i] = kNegInf;
        }
    }
  };
  auto row_max2 = [&]() __attribute__((always_inline)) {
    float mx = kNegInf;
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, fmaxf(sacc[0][i], sacc[1][i]));
    mx = fmaxf(mx, shfl_xor_f32(mx, 32));
    return mx * scale_log2;
  };
  // P~ = 2^(s c - m), rounded to bf16; rs = the lane's fp32 sum.
  auto expo = [&]() __attribute__((always_inline)) {
    float r4[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = fast_exp2(fmaf(sacc[t >> 1][8 * (t & 1) + e], scale_log2, -m2));
      r4[t] = ((x[0] + x[1]) + (x[2] + x[3])) + ((x[4] + x[5]) + (x[6] + x[7]));
      pb[t] = pack_bf16x8(x);
    }
    rs = (r4[0] + r4[1]) + (r4[2] + r4[3]);
  };
  // V(j): tile j's K at kt is read again only by the rare rescue.
  auto vph = [&](int j, const unsigned char* kt) __attribute__((always_inline)) {
    mask_tile(j);
    if (j == 0) m2 = row_max2();  // the reference: exact row max of tile 0 (key 0 is visible to every row)
    expo();
    if (__builtin_expect(__ballot(!(rs <= kSumLimit)) != 0, 0)) {
      // rare: move the reference to the exact running max and redo the tile
      __builtin_amdgcn_sched_barrier(0);
      scores(kt);
      mask_tile(j);
      const float mx2 = row_max2();
      const bool grow = mx2 > m2;
      const float alpha = grow ? fast_exp2(m2 - mx2) : 1.f;
      m2 = grow ? mx2 : m2;
      lsum *= alpha;
#pragma unroll
      for (int mt = 0; mt < D / 32; ++mt) oacc[mt] *= alpha;
      expo();
      __builtin_amdgcn_sched_barrier(0);
    }
    lsum += rs;
    // keep the packing in this phase (the barrier orders memory only)
    asm volatile("" : "+v"(pb[0]), "+v"(pb[1]), "+v"(pb[2]), "+v"(pb[3]));
  };

  // Q and tile 0 land before the first barrier; tiles 1-3 are issued after
  // the first products (a copy in flight there makes the compiler wait for
  // every load before them)
  wait_vm_at_most<0>();
  lds_barrier();
  if (!lead) lds_barrier();
  mph(sb0, sb0, false, true);
  // tiles past the last are empty copies into ring slots no step reads, so
  // the copies and the waits need no branches
  issue_tile(1, sb1);
  issue_tile(2, sb2);
  issue_tile(3, sb3);
  // tile 1 (tiles 2 and 3 may still be in flight)
  wait_vm_at_most<4>();
  lds_barrier();
  vph(0, sb0);
  // Tile j at cur, j-1 at prev; tile j+3 goes to far.
  auto step = [&](int j, const unsigned char* cur, const unsigned char* prev, unsigned char* far)
      __attribute__((always_inline)) {
    lds_barrier();
    issue_tile(j + 3, far);
    mph(cur, prev, true, true);
    // tile j+1 (tiles j+2 and j+3 may still be in flight)
    wait_vm_at_most<4>();
    lds_barrier();
    vph(j, cur);
  };
  // Causal: key tiles past the last one with a key visible to this
  // wavefront's rows are masked out for all of them; the wavefront stops
  // computing after that tile (nfull) and only copies and keeps the
  // workgroup's barrier count in the remaining steps.
  const int nfull = CAUSAL ? min(ntiles, (qw0 + 31) / kBc + 1) : ntiles;
  for (int j = 1; j < nfull; j += 5) {
    step(j, sb1, sb0, sb4);
    if (j + 1 < nfull) step(j + 1, sb2, sb1, sb0);
    if (j + 2 < nfull) step(j + 2, sb3, sb2, sb1);
    if (j + 3 < nfull) step(j + 3, sb4, sb3, sb2);
    if (j + 4 < nfull) step(j + 4, sb0, sb4, sb3);
  }
  auto slot = [&](int t) __attribute__((always_inline)) -> unsigned char* {
    t %= 5;
    return t == 0 ? sb0 : t == 1 ? sb1 : t == 2 ? sb2 : t == 3 ? sb3 : sb4;
  };
  if (CAUSAL && nfull < ntiles) {
    // the P~V product of tile nfull - 1 (its ring slot is overwritten only by
    // tile nfull + 4, issued at the second step below)
    lds_barrier();
    issue_tile(nfull + 3, slot(nfull + 3));
    mph(slot(nfull), slot(nfull - 1), true, false);
    wait_vm_at_most<4>();
    lds_barrier();
    for (int j = nfull + 1; j < ntiles; ++j) {
      lds_barrier();
      issue_tile(j + 3, slot(j + 3));
      wait_vm_at_most<4>();
      lds_barrier();
    }
    wait_vm_at_most<0>();  // the last (empty) copies land before the workgroup ends
    lds_barrier();
  } else {
    wait_vm_at_most<0>();  // the last (empty) copies land before the workgroup ends
    lds_barrier();
    mph(slot(ntiles - 1), slot(ntiles - 1), true, false);
  }
  if (lead) lds_barrier();

  const float lt = lsum + shfl_xor_f32(lsum, 32);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  const float lse2 = lt > 0.f ? m2 + fast_log2(lt) : kNegInf;
  if (qr < N) {
    __bf16* Oh = O + base;
    MergeWeights mw{0.f, 1.f, lse2 * kLn2};
    if constexpr (MERGE) mw = merge_weights(LSE[(int64_t)bh * N + qr], lse2);
#pragma unroll
    for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int d0 = 32 * mt + 8 * c + 4 * g;
        __bf16* dst = Oh + (int64_t)qr * D + d0;
        *reinterpret_cast<u32x2*>(dst) = merged_out4<MERGE>(dst, oacc[mt][4 * c] * inv, oacc[mt][4 * c + 1] * inv,
                                                            oacc[mt][4 * c + 2] * inv, oacc[mt][4 * c + 3] * inv, mw);
      }
    if (g == 0 && LSE != nullptr) LSE[(int64_t)bh * N + qr] = mw.lse;
  }
}

template <bool CAUSAL, bool MERGE>
hipError_t run_pp4(const FwdArgs& a, hipStream_t s) {
  constexpr int BR = 8 * 32;
  const int n_qtiles = (a.N + BR - 1) / BR;
  const int total = n_qtiles * a.B * a.H;
  hipLaunchKernelGGL((fwd_pp4_kernel<CAUSAL, MERGE>), dim3(total), dim3(512), 0, s, static_cast<const __bf16*>(a.q),
                     static_cast<const __bf16*>(a.k), static_cast<const __bf16*>(a.v),
                     static_cast<__bf16*>(a.o), a.lse, a.N, n_qtiles, total, a.scale * kLog2e);
  return hipGetLastError();
}

template <int D, int QT, int NBUF, bool CAUSAL, bool MERGE>
hipError_t run_bf16(const FwdArgs& a, hipStream_t s) {
  constexpr int BR = kWaves * 32 * QT;
  const int n_qtiles = (a.N + BR - 1) / BR;
  const int total = n_qtiles * a.B * a.H;
  const float scale_log2 = a.scale * kLog2e;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, QT, NBUF, CAUSAL, MERGE>), dim3(total), dim3(kThreads), 0, s,
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
  if (a.merge) {
    if (a.d == 64) return a.causal ? run_pp4<true, true>(a, s) : run_pp4<false, true>(a, s);
    return a.causal ? run_bf16<128, 1, 2, true, true>(a, s) : run_bf16<128, 1, 2, false, true>(a, s);
  }
  if (a.d == 64) return a.causal ? run_pp4<true, false>(a, s) : run_pp4<false, false>(a, s);
  return a.causal ? run_bf16<128, 1, 2, true, false>(a, s) : run_bf16<128, 1, 2, false, false>(a, s);
}

hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t s) {
  return a.causal ? run_f32<true>(a, s) : run_f32<false>(a, s);
}

}  // namespace attn
