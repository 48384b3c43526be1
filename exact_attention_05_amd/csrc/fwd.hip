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

template <int D, int QT, int NBUF, bool CAUSAL>
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
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      // rows past the end read row N-1 (valid memory); they are masked out
      const int row = min(kb + ld_key[i], N - 1);
      const int64_t off = (int64_t)row * D + ld_col[i];
      const int lds_line = 4 * (wave * NLD + i);
      global_to_lds16(Kh + off, kt + lds_line * 256);
      global_to_lds16(Vh + off, vt + lds_line * 256);
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

  // Epilogue: O = U / l (bf16, RNE) and LSE = (m + log2 l) * ln 2.
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
// Ping-pong variant.  Eight wavefronts, two per SIMD: wavefronts 0-3 lead and
// 4-7 trail by one phase.  Per K/V tile j a wavefront runs a matrix phase
// (S_j^T = K_j Q^T for the whole tile, then O^T += V_{j-1}^T P~_{j-1}^T) and
// a vector phase (mask, exponentials P~_j, row sums, reference check).  A
// workgroup barrier separates phases, so on every SIMD one wavefront issues
// matrix instructions while the other does the exponentials of its own tile,
// instead of both competing for the same unit.  The matrix-phase wavefront
// runs at raised issue priority so that its next product starts as soon as
// the matrix unit frees up.  Online state, reference rules and LDS layout
// are those of fwd_bf16_kernel; tile t's K is read in phases 2t and 2t+1,
// its V in phases 2t+2 and 2t+3, and tile t+2 is copied at phase 2t.
// ---------------------------------------------------------------------------
template <int D, int QT, bool CAUSAL>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) void fwd_pp_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    __bf16* __restrict__ O, float* __restrict__ LSE, int N, int n_qtiles, int total_wg,
    float scale_log2) {
  using T = TileLayout<D>;
  constexpr int NW = 8;
  constexpr int BR = NW * 32 * QT;
  constexpr int NCP = 2 * (D / 8) / NW;  // 1 KB copies per wavefront per tile
  static_assert(NCP >= 1 && NCP * NW == 2 * (D / 8), "tile copy split");
  __shared__ __attribute__((aligned(1024))) unsigned char sb0[2 * T::kBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char sb1[2 * T::kBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char sb2[2 * T::kBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char sb3[2 * T::kBytes];

  const int lid = xcd_remap(blockIdx.x, total_wg);
  const int bh = lid / n_qtiles;
  int qtile = lid % n_qtiles;
  if (CAUSAL) qtile = n_qtiles - 1 - qtile;  // longest rows first

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const bool lead = wave < 4;
  const int g = lane >> 5, l32 = lane & 31;
  const int64_t base = (int64_t)bh * N * D;
  const __bf16* Qh = Q + base;
  const __bf16* Kh = K + base;
  const __bf16* Vh = V + base;
  __bf16* Oh = O + base;

  const int q0 = qtile * BR;
  const int qw0 = q0 + wave * 32 * QT;
  const int kend = CAUSAL ? min(N, q0 + BR) : N;
  const int ntiles = (kend + kBc - 1) / kBc;

  int ld_key[NCP], ld_col[NCP], ld_dst[NCP];
  bool ld_v[NCP];
#pragma unroll
  for (int i = 0; i < NCP; ++i) {
    const int c = wave * NCP + i;
    const int cl = c % (D / 8);
    const int line = 4 * cl + (lane >> 4);
    int k, ch;
    T::at(line, lane & 15, k, ch);
    ld_key[i] = k;
    ld_col[i] = 8 * ch;
    ld_v[i] = c >= D / 8;
    ld_dst[i] = (ld_v[i] ? T::kBytes : 0) + 4 * cl * 256;
  }
  auto issue_tile_copy = [&](int kb, unsigned char* kt) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NCP; ++i) {
      const int row = min(kb + ld_key[i], N - 1);  // rows past the end are masked out
      const int64_t off = (int64_t)row * D + ld_col[i];
      global_to_lds16((ld_v[i] ? Vh : Kh) + off, kt + ld_dst[i]);
    }
  };

  issue_tile_copy(0, sb0);
  if (ntiles > 1) issue_tile_copy(kBc, sb1);

  bf16x8 qf[QT][D / 16];
#pragma unroll
  for (int nt = 0; nt < QT; ++nt) {
    const int qr = qw0 + nt * 32 + l32;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
      qf[nt][ks] = qr < N ? *reinterpret_cast<const bf16x8*>(Qh + (int64_t)qr * D + 16 * ks + 8 * g) : bf16x8{};
  }

  f32x16 oacc[QT][D / 32];
  float m2[QT], lsum[QT], rs[QT];
#pragma unroll
  for (int nt = 0; nt < QT; ++nt) {
    m2[nt] = kNegInf;
    lsum[nt] = 0.f;
#pragma unroll
    for (int mt = 0; mt < D / 32; ++mt) oacc[nt][mt] = f32x16{};
  }

  int koff[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) koff[ks] = T::offset(l32, 2 * ks + g);
  constexpr int kKhStep = 32 * D * 2;
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
  constexpr int kTStep = 16 * D * 2;

  f32x16 sacc[QT][2];  // S^T of the current tile, two halves of 32 keys
  bf16x8 pb[QT][4];    // P~ of the previous tile, four 16-key operands

  // S^T = K Q^T for the tile whose K is at kt (both halves).
  auto scores = [&](const unsigned char* kt) __attribute__((always_inline)) {
#pragma unroll
    for (int nt = 0; nt < QT; ++nt) sacc[nt][0] = sacc[nt][1] = f32x16{};
    bf16x8 a = *reinterpret_cast<const bf16x8*>(kt + koff[0]);
#pragma unroll
    for (int r = 0; r < 2 * (D / 16); ++r) {
      const int hh = r / (D / 16), ks = r % (D / 16);
      bf16x8 an = a;
      if (r + 1 < 2 * (D / 16)) {
        const int hn = (r + 1) / (D / 16), kn = (r + 1) % (D / 16);
        an = *reinterpret_cast<const bf16x8*>(kt + koff[kn] + hn * kKhStep);
      }
#pragma unroll
      for (int nt = 0; nt < QT; ++nt) sacc[nt][hh] = mfma32x32x16(a, qf[nt][ks], sacc[nt][hh]);
      a = an;
    }
  };
  // V^T operand of 16-key slice t, dims 32mt..+31 (two transposing reads).
  auto vop = [&](const unsigned char* vt, int t, int mt) __attribute__((always_inline)) {
    const u32x2 lo = lds_read_tr16(vt + voff[0][mt] + t * kTStep);
    const u32x2 hi = lds_read_tr16(vt + voff[1][mt] + t * kTStep);
    const u32x4 w = {lo[0], lo[1], hi[0], hi[1]};
    return bitcast<bf16x8>(w);
  };
  // Matrix phase of tile j: O^T += V_{j-1}^T P~_{j-1}^T (V at vt) first, so
  // that P~ dies before S_j^T = K_j Q^T (K at kt) is written; either part may
  // be absent (first and last phases).  Each operand is read one product
  // ahead of its use, so LDS latency overlaps the matrix unit.
  auto mphase = [&](const unsigned char* kt, const unsigned char* vt, bool do_pv, bool do_qk)
      __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(1);
    if (do_pv) {
      bf16x8 a = vop(vt, 0, 0);
#pragma unroll
      for (int r = 0; r < 4 * (D / 32); ++r) {
        const int t = r / (D / 32), mt = r % (D / 32);
        bf16x8 an = a;
        if (r + 1 < 4 * (D / 32)) an = vop(vt, (r + 1) / (D / 32), (r + 1) % (D / 32));
#pragma unroll
        for (int nt = 0; nt < QT; ++nt) oacc[nt][mt] = mfma32x32x16(a, pb[nt][t], oacc[nt][mt]);
        a = an;
      }
    }
    if (do_qk) scores(kt);
    __builtin_amdgcn_s_setprio(0);
  };

  // P~ = 2^(s*c - m) of query tile nt, rounded to bf16; rs = lane's fp32 sum.
  auto expo = [&](int nt) __attribute__((always_inline)) {
    float r4[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = fast_exp2(fmaf(sacc[nt][t >> 1][8 * (t & 1) + e], scale_log2, -m2[nt]));
      r4[t] = ((x[0] + x[1]) + (x[2] + x[3])) + ((x[4] + x[5]) + (x[6] + x[7]));
      pb[nt][t] = pack_bf16x8(x);
    }
    rs[nt] = (r4[0] + r4[1]) + (r4[2] + r4[3]);
  };

  auto mask_tile = [&](int j) __attribute__((always_inline)) {
    const int kb = j * kBc;
    if ((kb + kBc > N) || (CAUSAL && kb + kBc - 1 > qw0)) {
#pragma unroll
      for (int nt = 0; nt < QT; ++nt) {
        const int qr = qw0 + nt * 32 + l32;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = kb + 32 * hh + acc_row(i, g);
            const bool vis = key < N && (!CAUSAL || key <= qr);
            if (!vis) sacc[nt][hh][i] = kNegInf;
          }
      }
    }
  };
  auto row_max2 = [&](int nt) __attribute__((always_inline)) {
    float mx = kNegInf;
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, fmaxf(sacc[nt][0][i], sacc[nt][1][i]));
    mx = fmaxf(mx, shfl_xor_f32(mx, 32));
    return mx * scale_log2;
  };

  // Vector phase of tile j (K still in LDS at kt).  The scores die as the
  // exponentials are formed; the rare rescue recomputes them from K.
  auto vphase = [&](int j, const unsigned char* kt) __attribute__((always_inline)) {
    mask_tile(j);
    if (j == 0) {
      // the reference m: exact row max of tile 0 (key 0 is visible to every row)
#pragma unroll
      for (int nt = 0; nt < QT; ++nt) m2[nt] = row_max2(nt);
    }
#pragma unroll
    for (int nt = 0; nt < QT; ++nt) expo(nt);
    bool bad = false;
#pragma unroll
    for (int nt = 0; nt < QT; ++nt) bad |= !(rs[nt] <= kSumLimit);
    if (__builtin_expect(__ballot(bad) != 0, 0)) {
      __builtin_amdgcn_sched_barrier(0);
      scores(kt);
      mask_tile(j);
#pragma unroll
      for (int nt = 0; nt < QT; ++nt) {
        const float mx2 = row_max2(nt);
        const bool grow = mx2 > m2[nt];
        const float alpha = grow ? fast_exp2(m2[nt] - mx2) : 1.f;
        m2[nt] = grow ? mx2 : m2[nt];
        lsum[nt] *= alpha;
#pragma unroll
        for (int mt = 0; mt < D / 32; ++mt) oacc[nt][mt] *= alpha;
        expo(nt);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int nt = 0; nt < QT; ++nt) lsum[nt] += rs[nt];
  };

  auto phase_barrier = [&]() __attribute__((always_inline)) { lds_barrier(); };

  // One tile step = two phases.  kt: tile j's buffer, vprev: tile j-1's
  // buffer, next: where tile j+2 goes.
  auto tile_step = [&](int j, unsigned char* kt, unsigned char* vprev, unsigned char* next)
      __attribute__((always_inline)) {
    if (j + 1 < ntiles) wait_vm_at_most<NCP>(); else wait_vm_at_most<0>();
    phase_barrier();
    if (j + 2 < ntiles) issue_tile_copy((j + 2) * kBc, next);
    const unsigned char* vt = vprev + T::kBytes;
    if (lead) mphase(kt, vt, true, true);
    else vphase(j - 1, vprev);
    phase_barrier();
    if (lead) vphase(j, kt);
    else mphase(kt, vt, true, true);
  };

  // Tile 0: scores only.
  if (ntiles > 1) wait_vm_at_most<NCP>(); else wait_vm_at_most<0>();
  phase_barrier();
  if (ntiles > 2) issue_tile_copy(2 * kBc, sb2);
  if (lead) mphase(sb0, nullptr, false, true);
  phase_barrier();
  if (lead) vphase(0, sb0);
  else mphase(sb0, nullptr, false, true);
  for (int j = 1; j < ntiles; j += 4) {
    tile_step(j, sb1, sb0, sb3);
    if (j + 1 < ntiles) tile_step(j + 1, sb2, sb1, sb0); else break;
    if (j + 2 < ntiles) tile_step(j + 2, sb3, sb2, sb1); else break;
    if (j + 3 < ntiles) tile_step(j + 3, sb0, sb3, sb2); else break;
  }
  // Final phases: products of the last tile (ring slot (ntiles - 1) % 4).
  {
    const int tl = ntiles - 1;
    const unsigned char* kt = (tl & 3) == 0 ? sb0 : (tl & 3) == 1 ? sb1 : (tl & 3) == 2 ? sb2 : sb3;
    const unsigned char* vt = kt + T::kBytes;
    phase_barrier();
    if (lead) mphase(nullptr, vt, true, false);
    else vphase(tl, kt);
    phase_barrier();
    if (!lead) mphase(nullptr, vt, true, false);
  }

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

template <int D, int QT, int NBUF, bool CAUSAL>
hipError_t run_bf16(const FwdArgs& a, hipStream_t s) {
  constexpr int BR = kWaves * 32 * QT;
  const int n_qtiles = (a.N + BR - 1) / BR;
  const int total = n_qtiles * a.B * a.H;
  const float scale_log2 = a.scale * kLog2e;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, QT, NBUF, CAUSAL>), dim3(total), dim3(kThreads), 0, s,
                     static_cast<const __bf16*>(a.q), static_cast<const __bf16*>(a.k),
                     static_cast<const __bf16*>(a.v), static_cast<__bf16*>(a.o), a.lse, a.N, n_qtiles,
                     total, scale_log2);
  return hipGetLastError();
}

template <int D, int QT, bool CAUSAL>
hipError_t run_pp(const FwdArgs& a, hipStream_t s) {
  constexpr int BR = 8 * 32 * QT;
  const int n_qtiles = (a.N + BR - 1) / BR;
  const int total = n_qtiles * a.B * a.H;
  hipLaunchKernelGGL((fwd_pp_kernel<D, QT, CAUSAL>), dim3(total), dim3(512), 0, s,
                     static_cast<const __bf16*>(a.q), static_cast<const __bf16*>(a.k),
                     static_cast<const __bf16*>(a.v), static_cast<__bf16*>(a.o), a.lse, a.N, n_qtiles,
                     total, a.scale * kLog2e);
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
  if (a.d == 64) return a.causal ? run_pp<64, 2, true>(a, s) : run_pp<64, 2, false>(a, s);
  return a.causal ? run_bf16<128, 1, 2, true>(a, s) : run_bf16<128, 1, 2, false>(a, s);
}

hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t s) {
  return a.causal ? run_f32<true>(a, s) : run_f32<false>(a, s);
}

}  // namespace attn
