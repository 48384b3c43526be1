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
//                    streams 64-key tiles (K, V) through LDS:
//                    S^T = K Q^T, dP^T = V dO^T, dS^T = P^T o (dP^T - D),
//                    dQ^T += K^T dS^T.
// dK and dQ are multiplied by the softmax scale at the end (section 8.8.4).
// Causal, d = 64: a wavefront stops computing once the rest of its streamed
// tiles are hidden from it (dK/dV visits query tiles last first for this),
// and the two wavefronts of a SIMD own row blocks s and 7 - s, so every SIMD
// has the same share of the diagonal.
//
// Variant with atomic dQ (the single-pass alternative that section 8.8
// contrasts with the split into a dK/dV and a dQ kernel): bwd_dkdv also adds
// every tile's dS K into an fp32 dQ accumulator with atomic adds, and a
// final pass scales it into dQ.  The workgroup puts its dS tile in LDS as
// [key][query] and its K rows as [key][dim]; both go through the same
// transposing reads, so dQ = dS K contracts over the workgroup's 128 keys in
// one 32 x 32 output block per wavefront (two for d = 128), one atomic per
// element and workgroup.  The summation order then depends on timing, so
// this variant is not bitwise deterministic.
// Tiles go HBM -> LDS with direct-to-LDS copies into the swizzled tile layout
// of common.h, in a ring of buffers copied ahead of use.  Products that
// contract over the sequence take their P / dS operand straight from the
// accumulator of the previous product, and their other operand from the same
// tile through transposing LDS reads whose 4-row chunks follow the
// accumulator's row order (the scheme of V^T in the forward).
#include "common.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kT = 64;  // rows per streamed tile

// Logical work id -> (head, tile).  Heads are taken in groups of `group`
// (the host picks about one eighth of them, one group per XCD share of the
// grid); inside a group the ids run tile-major, so with causal masking the
// heaviest tiles of all the group's heads start first and the light ones
// fill the tail.
__device__ __forceinline__ void head_tile(int lid, int n_tiles, int BH, int group, int& bh, int& tile) {
  const int gi = lid / (group * n_tiles);
  const int gsz = min(group, BH - gi * group);
  const int r = lid - gi * group * n_tiles;
  tile = r / gsz;
  bh = gi * group + r % gsz;
}

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
// Per-row terms, written to the workspace:
//   delta[r] = D_r = rowsum(dO o O)_r                      (fp32)
//   nl2[r]   = -LSE_r * log2(e)                           (fp32)
//   dsplit[r]= (h, m, l, 0) in bf16 with h + m + l = -D_r to about 2^-24
//              relative: each part is the bf16 rounding of what the previous
//              parts left, and every remainder is exact in fp32.
//   lsplit[r]= the same split of nl2[r] / (scale log2 e).
// A split lets an MFMA add its value to a whole row of a product: one extra
// K-slice with (h, m, l) on the row side and (1, 1, 1) on the column side.
// dP - D comes out that way, and so does S + nl2 / (scale log2 e), whose
// product with scale log2 e is the exponent of P.
// ---------------------------------------------------------------------------
__device__ __forceinline__ u32x2 split3_bf16(float x) {
  const __bf16 h = (__bf16)x;
  const float r1 = x - (float)h;
  const __bf16 m = (__bf16)r1;
  const __bf16 l = (__bf16)(r1 - (float)m);
  const bf16x2 hm = {h, m};
  const bf16x2 l0 = {l, (__bf16)0.f};
  return u32x2{bitcast<uint32_t>(hm), bitcast<uint32_t>(l0)};
}

template <int D>
__global__ __launch_bounds__(kThreads) void bwd_preprocess_kernel(const __bf16* __restrict__ O,
                                                                  const __bf16* __restrict__ dO,
                                                                  const float* __restrict__ LSE,
                                                                  float* __restrict__ delta, float* __restrict__ nl2,
                                                                  u32x2* __restrict__ dsplit, u32x2* __restrict__ lsplit,
                                                                  float scale_log2, int64_t rows) {
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
  if (row < rows && u == 0) {
    const float l2 = -LSE[row] * kLog2e;
    delta[row] = acc;
    nl2[row] = l2;
    dsplit[row] = split3_bf16(-acc);
    lsplit[row] = split3_bf16(l2 / scale_log2);
  }
}

// ---------------------------------------------------------------------------
// dK, dV: key tiles outer.  LDS buffer: Q tile | dO tile | nl2[64] | dsplit[64].
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL, bool ATOMIC_DQ = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(D == 64 ? 2 : 1))) void bwd_dkdv_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const __bf16* __restrict__ dO, const float* __restrict__ nl2, const u32x2* __restrict__ dsplit,
    __bf16* __restrict__ dK, __bf16* __restrict__ dV, float* __restrict__ dqacc, int N, int BH, int n_ktiles,
    int group, float scale, float scale_log2) {
  using T = TileLayout<D>;
  using TX = TileLayout<64>;  // dS tile of the atomic-dQ variant: [128 keys][64 queries]
  constexpr int BK = kWaves * 32;
  constexpr int NB = D == 64 ? 4 : 2;  // ring depth; tiles are copied NB/2 ahead
  constexpr int kBuf = 2 * T::kBytes + kT * 4 + kT * 8;
  __shared__ __attribute__((aligned(1024))) unsigned char sb0[kBuf];
  __shared__ __attribute__((aligned(1024))) unsigned char sb1[kBuf];
  __shared__ __attribute__((aligned(1024))) unsigned char sb2[NB > 2 ? kBuf : 16];
  __shared__ __attribute__((aligned(1024))) unsigned char sb3[NB > 2 ? kBuf : 16];
  // atomic-dQ variant: the workgroup's K rows and the dS of two tiles (the
  // dS of tile s is contracted at step s + 1, while tile s + 1 fills the
  // other buffer)
  __shared__ __attribute__((aligned(1024))) unsigned char skt[ATOMIC_DQ ? 2 * T::kBytes : 16];
  __shared__ __attribute__((aligned(1024))) unsigned char sx0[ATOMIC_DQ ? 2 * TX::kBytes : 16];
  __shared__ __attribute__((aligned(1024))) unsigned char sx1[ATOMIC_DQ ? 2 * TX::kBytes : 16];

  int bh, ktile;  // key tile 0 has the most query tiles under causal masking
  head_tile(xcd_remap(blockIdx.x, BH * n_ktiles), n_ktiles, BH, group, bh, ktile);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, held in an SGPR
  const int g = lane >> 5, l32 = lane & 31;
  const int64_t base = (int64_t)bh * N * D;
  const int k0 = ktile * BK;
  const int kw0 = k0 + wave * 32;
  const int key = kw0 + l32;

  const TileCopy<D, kWaves> cp(wave, lane);
  const TileOffsets<D> of(lane);
  const float* nl2h = nl2 + (int64_t)bh * N;
  const uint32_t* dsh = reinterpret_cast<const uint32_t*>(dsplit + (int64_t)bh * N);
  // wavefront 0 copies the tile's nl2 (64 words), wavefronts 1 and 2 its
  // dsplit (2 words per row, 32 rows each)
  auto issue_tile = [&](int it, unsigned char* buf) __attribute__((always_inline)) {
    const int q0 = it * kT;
    cp.issue(Q + base, q0, N, buf);
    cp.issue(dO + base, q0, N, buf + T::kBytes);
    if (wave == 0) {
      global_to_lds4(nl2h + min(q0 + lane, N - 1), buf + 2 * T::kBytes);
    } else if (wave < 3) {
      const int w = 64 * (wave - 1) + lane;
      const int r = min(q0 + (w >> 1), N - 1);
      global_to_lds4(dsh + 2 * r + (w & 1), buf + 2 * T::kBytes + kT * 4 + 256 * (wave - 1));
    }
  };
  // direct-to-LDS copies issued per wavefront per tile
  constexpr int kCopies = 2 * TileCopy<D, kWaves>::kPerWave;

  const int i_begin = CAUSAL ? k0 / kT : 0;
  const int i_end = (N + kT - 1) / kT;
  const int ntiles = i_end - i_begin;
  constexpr int A = NB / 2;
  // the K rows first: they are older than every tile copy, so the first
  // tile's wait covers them
  if constexpr (ATOMIC_DQ) {
    cp.issue(K + base, k0, N, skt);
    cp.issue(K + base, k0 + kT, N, skt + T::kBytes);
  }
#pragma unroll
  for (int p = 0; p < A; ++p)
    if (p < ntiles) issue_tile(i_begin + p, p == 0 ? sb0 : sb1);

  // K, V of this wavefront's 32 keys as B operands: lane holds row `key`, dims 16ks + 8g .. +7
  bf16x8 kB[D / 16], vB[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    kB[ks] = key < N ? *reinterpret_cast<const bf16x8*>(K + base + (int64_t)key * D + 16 * ks + 8 * g) : bf16x8{};
    vB[ks] = key < N ? *reinterpret_cast<const bf16x8*>(V + base + (int64_t)key * D + 16 * ks + 8 * g) : bf16x8{};
  }
  // column side of the -D slice: (1, 1, 1) in the first K-group, zero in the second
  const bf16x8 ones3 = bitcast<bf16x8>(g == 0 ? u32x4{0x3F803F80u, 0x3F80u, 0u, 0u} : u32x4{0u, 0u, 0u, 0u});
  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int mt = 0; mt < D / 32; ++mt) dk[mt] = dv[mt] = f32x16{};

  // atomic-dQ variant: this lane's row of a dS tile (key kw0 + l32)
  const int xr = wave * 32 + l32;
  const int xrow = (xr >> 6) * TX::kBytes;
  auto compute = [&](int it, const unsigned char* buf, unsigned char* xt) __attribute__((always_inline)) {
    unsigned char* const xrp = xt + xrow;
    const int q0 = it * kT;
    if (CAUSAL && q0 + kT - 1 < kw0) {  // every query of the tile is above this wavefront's keys
      if constexpr (ATOMIC_DQ) {
#pragma unroll
        for (int c = 0; c < 8; ++c) *reinterpret_cast<u32x4*>(xrp + TX::offset(xr & 63, c)) = u32x4{};
      }
      return;
    }
    const unsigned char* Qt = buf;
    const unsigned char* Dt = buf + T::kBytes;
    const float* ls = reinterpret_cast<const float*>(buf + 2 * T::kBytes);
    const u32x2* dsl = reinterpret_cast<const u32x2*>(buf + 2 * T::kBytes + kT * 4);
    // keys past N only matter where dS leaves the workgroup (atomic dQ)
    const bool need_mask = (q0 + kT > N) || (CAUSAL && q0 < kw0 + 31) || (ATOMIC_DQ && kw0 + 32 > N);
    // the two 32-query halves one after the other, so that only one pair of
    // score accumulators is live
#pragma unroll
    for (int qh = 0; qh < 2; ++qh) {
      __builtin_amdgcn_sched_barrier(0);  // keep the halves apart in the schedule
      f32x16 sacc = {}, dpacc = {};
      // dP - D: the row side of the extra slice is query row 32qh + l32's split of -D
      const u32x2 dw = dsl[32 * qh + l32];
      dpacc = mfma32x32x16(bitcast<bf16x8>(u32x4{dw[0], dw[1], 0u, 0u}), ones3, dpacc);
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        sacc = mfma32x32x16(of.row(Qt, ks, qh), kB[ks], sacc);
        dpacc = mfma32x32x16(of.row(Dt, ks, qh), vB[ks], dpacc);
      }
      __builtin_amdgcn_sched_barrier(0);
      // lane holds queries q0 + 32qh + acc_row(i, g) of key `key`; hidden
      // pairs get S = -inf, hence P = 0 and dS = 0
      if (need_mask) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int qi = q0 + 32 * qh + acc_row(i, g);
          if (qi >= N || (CAUSAL && key > qi) || (ATOMIC_DQ && key >= N)) sacc[i] = kNegInf;
        }
      }
      // P = exp2(S*c - LSE*log2e), dS = P o (dP - D)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(ls + 32 * qh + 8 * c + 4 * g);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 4 * c + r;
          const float p = fast_exp2(fmaf(sacc[i], scale_log2, l4[r]));
          sacc[i] = p;
          dpacc[i] = p * dpacc[i];
        }
      }
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        float x[8], y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          x[e] = sacc[8 * tt + e];
          y[e] = dpacc[8 * tt + e];
        }
        const bf16x8 pb = pack_bf16x8(x);
        const bf16x8 sbf = pack_bf16x8(y);
#pragma unroll
        for (int mt = 0; mt < D / 32; ++mt) {
          dv[mt] = mfma32x32x16(of.tr(Dt, 2 * qh + tt, mt), pb, dv[mt]);
          dk[mt] = mfma32x32x16(of.tr(Qt, 2 * qh + tt, mt), sbf, dk[mt]);
        }
        if constexpr (ATOMIC_DQ) {
          // dS of queries 32qh + 16tt + 4g + 0..3 and +8 (the accumulator's
          // row order) into the lane's row of the dS tile
          const u32x4 w = bitcast<u32x4>(sbf);
          *reinterpret_cast<u32x2*>(xrp + TX::offset(xr & 63, 4 * qh + 2 * tt) + 8 * g) = u32x2{w[0], w[1]};
          *reinterpret_cast<u32x2*>(xrp + TX::offset(xr & 63, 4 * qh + 2 * tt + 1) + 8 * g) = u32x2{w[2], w[3]};
        }
      }
    }
  };

  // atomic-dQ variant: dQ[q0 .. q0+63] += dS K over the workgroup's keys.
  // Wavefront w owns query rows 32(w & 1) .. +31 and dims 32(w >> 1) .. +31
  // (and +64 for d = 128); both operands are transposing reads in the same
  // key order, the result lands with one fp32 atomic add per element.
  const TileOffsets<64> ox(lane);
  auto dq_tile = [&](int it, const unsigned char* xt) __attribute__((always_inline)) {
    const int q0 = it * kT;
    const int qb = 32 * (wave & 1);
#pragma unroll
    for (int nb = 0; nb < D / 64; ++nb) {
      const int mtk = (wave >> 1) + 2 * nb;
      f32x16 acc = {};
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk)
        acc = mfma32x32x16(ox.tr(xt + (kk >> 2) * TX::kBytes, kk & 3, qb >> 5),
                           of.tr(skt + (kk >> 2) * T::kBytes, kk & 3, mtk), acc);
      float* dst = dqacc + ((int64_t)bh * N + q0 + qb) * D + 32 * mtk + l32;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = acc_row(i, g);
        if (q0 + qb + r < N) atomicAdd(dst + (int64_t)r * D, acc[i]);
      }
    }
  };

  // Tile s of the sweep (query tile i_begin + s) is in buffer s % NB; at its
  // step the copies of tile s + A go to buffer (s + A) % NB, which held tile
  // s - A (NB = 2A) and is free after the barrier.
  // (Atomic dQ: the dS of tile s - 1, complete since the barrier, is
  // contracted and added before tile s is computed, so the adds are in flight
  // during that work.  The copy waits below count only tile copies: a wait
  // for tile s cannot pass before it lands, since loads complete in order and
  // the adds only raise the count.)
  auto step = [&](int s, const unsigned char* buf, unsigned char* next, unsigned char* xcur,
                  const unsigned char* xprev) __attribute__((always_inline)) {
    if (s + A - 1 < ntiles) {
      if (wave < 3) wait_vm_at_most<(A - 1) * (kCopies + 1)>(); else wait_vm_at_most<(A - 1) * kCopies>();
    } else {
      wait_vm_at_most<0>();
    }
    lds_barrier();
    if (s + A < ntiles) issue_tile(i_begin + s + A, next);
    if constexpr (ATOMIC_DQ) {
      if (s >= 1 && s - 1 < ntiles) dq_tile(i_begin + s - 1, xprev);
    }
    if (s < ntiles) compute(i_begin + s, buf, xcur);
  };
  // one exit per loop (steps past the end only wait and synchronise), so the
  // accumulators keep their registers across iterations
  if constexpr (NB == 4) {
    for (int s = 0; s < ntiles; s += 4) {
      step(s, sb0, sb2, sx0, sx1);
      step(s + 1, sb1, sb3, sx1, sx0);
      step(s + 2, sb2, sb0, sx0, sx1);
      step(s + 3, sb3, sb1, sx1, sx0);
    }
  } else {
    for (int s = 0; s < ntiles; s += 2) {
      step(s, sb0, sb1, sx0, sx1);
      step(s + 1, sb1, sb0, sx1, sx0);
    }
  }
  if constexpr (ATOMIC_DQ) {
    // the last tile's dS when the loop ended on it (its index is odd)
    if (ntiles % NB == 0) {
      lds_barrier();
      dq_tile(i_begin + ntiles - 1, sx1);
    }
  }

  if (key < N) {
    store_transposed_acc<D>(dV + base + (int64_t)key * D, dv, g, 1.f);
    store_transposed_acc<D>(dK + base + (int64_t)key * D, dk, g, scale);
  }
}

// ---------------------------------------------------------------------------
// dQ: query tiles outer.  LDS buffer: K tile | V tile.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(D == 64 ? 2 : 1))) void bwd_dq_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                                                          const __bf16* __restrict__ V,
                                                          const __bf16* __restrict__ dO,
                                                          const float* __restrict__ nl2,
                                                          const u32x2* __restrict__ dsplit, __bf16* __restrict__ dQ,
                                                          int N, int BH, int n_qtiles, int group, float scale,
                                                          float scale_log2) {
  using T = TileLayout<D>;
  constexpr int BQ = kWaves * 32;
  constexpr int NB = D == 64 ? 4 : 2;
  constexpr int kBuf = 2 * T::kBytes;
  __shared__ __attribute__((aligned(1024))) unsigned char sb0[kBuf];
  __shared__ __attribute__((aligned(1024))) unsigned char sb1[kBuf];
  __shared__ __attribute__((aligned(1024))) unsigned char sb2[NB > 2 ? kBuf : 16];
  __shared__ __attribute__((aligned(1024))) unsigned char sb3[NB > 2 ? kBuf : 16];

  int bh, qtile;
  head_tile(xcd_remap(blockIdx.x, BH * n_qtiles), n_qtiles, BH, group, bh, qtile);
  if (CAUSAL) qtile = n_qtiles - 1 - qtile;  // the last query tile sees the most keys
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, held in an SGPR
  const int g = lane >> 5, l32 = lane & 31;
  const int64_t base = (int64_t)bh * N * D;
  const int q0 = qtile * BQ;
  const int qw0 = q0 + wave * 32;
  const int qr = qw0 + l32;

  const TileCopy<D, kWaves> cp(wave, lane);
  const TileOffsets<D> of(lane);
  auto issue_tile = [&](int j, unsigned char* buf) __attribute__((always_inline)) {
    cp.issue(K + base, j * kT, N, buf);
    cp.issue(V + base, j * kT, N, buf + T::kBytes);
  };
  constexpr int kCopies = 2 * TileCopy<D, kWaves>::kPerWave;

  const int kend = CAUSAL ? min(N, q0 + BQ) : N;
  const int ntiles = (kend + kT - 1) / kT;
  constexpr int A = NB / 2;
#pragma unroll
  for (int p = 0; p < A; ++p)
    if (p < ntiles) issue_tile(p, p == 0 ? sb0 : sb1);

  bf16x8 qB[D / 16], doB[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    qB[ks] = qr < N ? *reinterpret_cast<const bf16x8*>(Q + base + (int64_t)qr * D + 16 * ks + 8 * g) : bf16x8{};
    doB[ks] = qr < N ? *reinterpret_cast<const bf16x8*>(dO + base + (int64_t)qr * D + 16 * ks + 8 * g) : bf16x8{};
  }
  const float nlse2 = qr < N ? nl2[(int64_t)bh * N + qr] : kNegInf;
  // -D slice: this lane's query split of -D in the first K-group (zero in the
  // second) against a row side of ones
  const u32x2 dw = qr < N ? dsplit[(int64_t)bh * N + qr] : u32x2{0u, 0u};
  const bf16x8 ndB = bitcast<bf16x8>(g == 0 ? u32x4{dw[0], dw[1], 0u, 0u} : u32x4{0u, 0u, 0u, 0u});
  const bf16x8 ones3 = bitcast<bf16x8>(u32x4{0x3F803F80u, 0x3F80u, 0u, 0u});

  f32x16 dq[D / 32];
#pragma unroll
  for (int mt = 0; mt < D / 32; ++mt) dq[mt] = f32x16{};

  auto compute = [&](int j, const unsigned char* buf) __attribute__((always_inline)) {
    const int kb = j * kT;
    if (CAUSAL && kb > qw0 + 31) return;  // every key of the tile is after this wavefront's queries
    const unsigned char* Kt = buf;
    const unsigned char* Vt = buf + T::kBytes;
    const bool need_mask = (kb + kT > N) || (CAUSAL && kb + kT - 1 > qw0);
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      __builtin_amdgcn_sched_barrier(0);  // keep the halves apart in the schedule
      f32x16 sacc = {};
      f32x16 dpacc = mfma32x32x16(ones3, ndB, f32x16{});
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        sacc = mfma32x32x16(of.row(Kt, ks, kh), qB[ks], sacc);
        dpacc = mfma32x32x16(of.row(Vt, ks, kh), doB[ks], dpacc);
      }
      __builtin_amdgcn_sched_barrier(0);
      // lane holds keys kb + 32kh + acc_row(i, g) of query qr
      if (need_mask) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kk = kb + 32 * kh + acc_row(i, g);
          if (kk >= N || (CAUSAL && kk > qr)) sacc[i] = kNegInf;
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = fast_exp2(fmaf(sacc[i], scale_log2, nlse2));
        dpacc[i] = p * dpacc[i];
      }
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        float y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = dpacc[8 * tt + e];
        const bf16x8 sbf = pack_bf16x8(y);
#pragma unroll
        for (int mt = 0; mt < D / 32; ++mt) dq[mt] = mfma32x32x16(of.tr(Kt, 2 * kh + tt, mt), sbf, dq[mt]);
      }
    }
  };

  auto step = [&](int s, const unsigned char* buf, unsigned char* next) __attribute__((always_inline)) {
    if (s + A - 1 < ntiles) wait_vm_at_most<(A - 1) * kCopies>(); else wait_vm_at_most<0>();
    lds_barrier();
    if (s + A < ntiles) issue_tile(s + A, next);
    if (s < ntiles) compute(s, buf);
  };
  if constexpr (NB == 4) {
    for (int s = 0; s < ntiles; s += 4) {
      step(s, sb0, sb2);
      step(s + 1, sb1, sb3);
      step(s + 2, sb2, sb0);
      step(s + 3, sb3, sb1);
    }
  } else {
    for (int s = 0; s < ntiles; s += 2) {
      step(s, sb0, sb1);
      step(s + 1, sb1, sb0);
    }
  }

  if (qr < N) store_transposed_acc<D>(dQ + base + (int64_t)qr * D, dq, g, scale);
}

// ---------------------------------------------------------------------------
// d = 64: ping-pong variants.  Eight wavefronts, two per SIMD; each owns 32
// keys (dK/dV) or 32 queries (dQ) and walks the streamed tiles in 32-row
// halves.  Per half h it runs a matrix phase M(h) -- the score products of
// half h, then the contraction of half h-1 into its accumulators -- and a
// vector phase V(h) -- mask, exponentials, dS, bf16 packing, plus the LDS
// reads of the row operands M(h+1) needs.  Every wavefront runs the same
// sequence M(0) V(0) M(1) V(1) ... with a workgroup barrier between phases;
// wavefronts 4-7 (trail) pass one extra barrier before starting and
// wavefronts 0-3 (lead) one after finishing, so each trail wavefront runs one
// phase behind the lead wavefront on its SIMD and the SIMD has one wavefront
// issuing MFMAs while the other issues VALU work.  M(h) issues its
// transposing reads first; they land while the score MFMAs run.
//
// Ring of 4 tile buffers: the copy of tile s+2 is issued at M(2s).  Each
// wavefront waits for its own copies of tile s+1 before the barrier that
// opens its M(2s+1); the trail's such barrier is the one that opens the
// lead's V(2s+1), the first reader of tile s+1.  The last reader of tile s is
// the trail's M(2s+2), well before tile s+4 is issued.
// ---------------------------------------------------------------------------
constexpr int kPPWaves = 8;
constexpr int kPPThreads = kPPWaves * 64;

template <bool CAUSAL>
__global__ __launch_bounds__(kPPThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_dkdv_pp_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const __bf16* __restrict__ dO, const u32x2* __restrict__ lsplit, const u32x2* __restrict__ dsplit,
    __bf16* __restrict__ dK, __bf16* __restrict__ dV, int N, int BH, int n_ktiles, int group, float scale,
    float scale_log2) {
  constexpr int D = 64;
  using T = TileLayout<D>;
  constexpr int NW = kPPWaves;
  constexpr int BK = NW * 32;
  constexpr int kBuf = 2 * T::kBytes + 2 * kT * 8;  // Q | dO | dsplit | lsplit
  __shared__ __attribute__((aligned(1024))) unsigned char sb0[kBuf];
  __shared__ __attribute__((aligned(1024))) unsigned char sb1[kBuf];
  __shared__ __attribute__((aligned(1024))) unsigned char sb2[kBuf];
  __shared__ __attribute__((aligned(1024))) unsigned char sb3[kBuf];

  int bh, ktile;
  head_tile(xcd_remap(blockIdx.x, BH * n_ktiles), n_ktiles, BH, group, bh, ktile);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool lead = wave < 4;
  const int g = lane >> 5, l32 = lane & 31;
  const int64_t base = (int64_t)bh * N * D;
  const int k0 = ktile * BK;
  // the lead and the trail wavefront of SIMD s (w = s and w = s + 4) own key
  // blocks s and 7 - s, so on a causal diagonal every SIMD has the same work
  const int kw0 = k0 + 32 * (wave < 4 ? wave : 11 - wave);
  const int key = kw0 + l32;

  const TileCopyBuf<D, NW> cp(wave, lane);
  const TileOffsets<D> of(lane);
  // wavefronts 0-1 copy the tile's dsplit, 2-3 its lsplit (2 words per row, 32 rows each)
  const uint32_t* sph = reinterpret_cast<const uint32_t*>((wave < 2 ? dsplit : lsplit) + (int64_t)bh * N);
  auto issue_tile = [&](int it, unsigned char* buf) __attribute__((always_inline)) {
    const int q0 = it * kT;
    cp.issue(Q + base, N, q0, buf);
    cp.issue(dO + base, N, q0, buf + T::kBytes);
    if (wave < 4) {
      const int w = 64 * (wave & 1) + lane;
      const int r = min(q0 + (w >> 1), N - 1);
      global_to_lds4(sph + 2 * r + (w & 1), buf + 2 * T::kBytes + 256 * wave);
    }
  };
  constexpr int kCopies = 2 * TileCopyBuf<D, NW>::kPerWave;
  // wait for this wavefront's copies of all tiles but the newest one
  // (one_after) or of all tiles
  auto wait_copies = [&](bool one_after) __attribute__((always_inline)) {
    if (one_after) {
      if (wave < 4) wait_vm_at_most<kCopies + 1>(); else wait_vm_at_most<kCopies>();
    } else {
      wait_vm_at_most<0>();
    }
  };

  const int i_begin = CAUSAL ? k0 / kT : 0;
  const int i_end = (N + kT - 1) / kT;
  const int ntiles = i_end - i_begin;
  // causal: query tiles are visited last first, so that on the diagonal the
  // tiles hidden from a wavefront's keys come at the end of its sequence;
  // positions past the sequence name the empty tile at i_end
  auto tidx = [&](int s) __attribute__((always_inline)) {
    return CAUSAL ? (s < ntiles ? i_end - 1 - s : i_end) : i_begin + s;
  };
  // this wavefront's K and V rows first, then the first tile (loads
  // complete in issue order)
  bf16x8 kB[D / 16], vB[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    kB[ks] = key < N ? *reinterpret_cast<const bf16x8*>(K + base + (int64_t)key * D + 16 * ks + 8 * g) : bf16x8{};
    vB[ks] = key < N ? *reinterpret_cast<const bf16x8*>(V + base + (int64_t)key * D + 16 * ks + 8 * g) : bf16x8{};
  }
  issue_tile(tidx(0), sb0);
  const bf16x8 ones3 = bitcast<bf16x8>(g == 0 ? u32x4{0x3F803F80u, 0x3F80u, 0u, 0u} : u32x4{0u, 0u, 0u, 0u});
  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int mt = 0; mt < D / 32; ++mt) dk[mt] = dv[mt] = f32x16{};
  f32x16 sacc, dpacc;             // S and dP - D of the current half
  bf16x8 pb[2], sbf[2];           // P and dS of the previous half, bf16
  bf16x8 rq[D / 16], rd[D / 16];  // Q and dO rows of the next half
  u32x2 dw, lw;                   // its splits of -D and of nl2 / (scale log2 e)

  auto read_rows = [&](const int QH, const unsigned char* buf) __attribute__((always_inline)) {
    dw = reinterpret_cast<const u32x2*>(buf + 2 * T::kBytes)[32 * QH + l32];
    lw = reinterpret_cast<const u32x2*>(buf + 2 * T::kBytes + kT * 8)[32 * QH + l32];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      rq[ks] = of.row(buf, ks, QH);
      rd[ks] = of.row(buf + T::kBytes, ks, QH);
    }
  };

  // M: S + nl2 / (scale log2 e) and dP - D of the current half (rows read
  // by the previous phase), then dV^T += dO^T P, dK^T += Q^T dS of the
  // previous half (tile at bprev, half 1 - QH).
  auto mph = [&](const int QH, const unsigned char* bprev, const bool do_acc, const bool do_scores)
      __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(1);
    const int QP = 1 - QH;
    bf16x8 tq[2][D / 32], td[2][D / 32];
    if (do_acc) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int mt = 0; mt < D / 32; ++mt) {
          td[tt][mt] = of.tr(bprev + T::kBytes, 2 * QP + tt, mt);
          tq[tt][mt] = of.tr(bprev, 2 * QP + tt, mt);
        }
    }
    if (do_scores) {
      dpacc = mfma32x32x16(bitcast<bf16x8>(u32x4{dw[0], dw[1], 0u, 0u}), ones3, f32x16{});
      sacc = mfma32x32x16(bitcast<bf16x8>(u32x4{lw[0], lw[1], 0u, 0u}), ones3, f32x16{});
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        sacc = mfma32x32x16(rq[ks], kB[ks], sacc);
        dpacc = mfma32x32x16(rd[ks], vB[ks], dpacc);
      }
    }
    if (do_acc) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int mt = 0; mt < D / 32; ++mt) {
          dv[mt] = mfma32x32x16(td[tt][mt], pb[tt], dv[mt]);
          dk[mt] = mfma32x32x16(tq[tt][mt], sbf[tt], dk[mt]);
        }
    }
    if (do_acc && do_scores) {
      __builtin_amdgcn_sched_group_barrier(0x0100, 8 * (D / 32), 0);
      __builtin_amdgcn_sched_group_barrier(0x0008, 2 + 2 * (D / 16) + 4 * (D / 32), 0);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // V: P = exp2((S + nl2 / c) c) with c = scale log2 e (0 where hidden),
  // dS = P o (dP - D) for the queries qa .. qa+31, packed to bf16; the rows
  // of the next half are read meanwhile (from bnext, half NQH).
  auto vph = [&](int qa, const bool next, const int NQH, const unsigned char* bnext)
      __attribute__((always_inline)) {
    if (next) read_rows(NQH, bnext);
    if ((qa + 31 >= N) || (CAUSAL && qa < kw0 + 31)) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int qi = qa + acc_row(i, g);
        if (qi >= N || (CAUSAL && key > qi)) sacc[i] = kNegInf;
      }
    }
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      float x[8], y[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int i = 8 * tt + e;
        const float p = fast_exp2(sacc[i] * scale_log2);
        x[e] = p;
        y[e] = p * dpacc[i];
      }
      pb[tt] = pack_bf16x8(x);
      sbf[tt] = pack_bf16x8(y);
    }
    // keep the packing in this phase (the barrier orders memory only)
    asm volatile("" : "+v"(pb[0]), "+v"(pb[1]), "+v"(sbf[0]), "+v"(sbf[1]));
  };

  // Tile 0.
  // the first tile before the first barrier; the next two go out after the
  // first products (a copy in flight there makes the compiler wait for every
  // load)
  wait_vm_at_most<0>();
  lds_barrier();
  if (!lead) lds_barrier();
  read_rows(0, sb0);
  mph(0, sb0, false, true);
  // tiles past the last are empty copies into ring slots no step reads,
  // so the copies and the waits need no branches
  issue_tile(tidx(1), sb1);
  issue_tile(tidx(2), sb2);
  lds_barrier();
  vph(tidx(0) * kT, true, 1, sb0);
  wait_copies(true);
  lds_barrier();
  mph(1, sb0, true, true);
  lds_barrier();
  vph(tidx(0) * kT + 32, ntiles > 1, 0, sb1);
  lds_barrier();
  // Tile s >= 1 at cur, s-1 at prev, s+1 at nxt1; tile s+2 goes to nxt2.
  auto step = [&](int s, const unsigned char* cur, const unsigned char* prev, const unsigned char* nxt1,
                  unsigned char* nxt2) __attribute__((always_inline)) {
    const int q0 = tidx(s) * kT;
    issue_tile(tidx(s + 2), nxt2);
    mph(0, prev, true, true);
    lds_barrier();
    vph(q0, true, 1, cur);
    wait_copies(true);
    lds_barrier();
    mph(1, cur, true, true);
    lds_barrier();
    vph(q0 + 32, s + 1 < ntiles, 0, nxt1);
    lds_barrier();
  };
  // Causal: query tiles before the first one with a query that sees this
  // wavefront's keys (the last ones visited) are masked out for all of
  // them; the wavefront stops computing after the first (nfull) and only
  // copies and keeps the workgroup's barrier count in the remaining steps.
  const int nfull = CAUSAL ? max(1, min(ntiles, i_end - kw0 / kT)) : ntiles;
  for (int s = 1; s < nfull; s += 4) {
    step(s, sb1, sb0, sb2, sb3);
    if (s + 1 < nfull) step(s + 1, sb2, sb1, sb3, sb0);
    if (s + 2 < nfull) step(s + 2, sb3, sb2, sb0, sb1);
    if (s + 3 < nfull) step(s + 3, sb0, sb3, sb1, sb2);
  }
  auto slot = [&](int t) __attribute__((always_inline)) -> unsigned char* {
    t &= 3;
    return t == 0 ? sb0 : t == 1 ? sb1 : t == 2 ? sb2 : sb3;
  };
  // contraction of the last half of tile position nfull - 1 (its ring slot is
  // overwritten only by position nfull + 3, issued at the second step below)
  if (CAUSAL && nfull < ntiles) {
    for (int s = nfull; s < ntiles; ++s) {
      issue_tile(tidx(s + 2), slot(s + 2));
      if (s == nfull) mph(0, slot(nfull - 1), true, false);
      lds_barrier();
      wait_copies(true);
      lds_barrier();
      lds_barrier();
      lds_barrier();
    }
  } else {
    mph(0, slot(ntiles - 1), true, false);
  }
  if (lead) lds_barrier();
  wait_vm_at_most<0>();  // the last (empty) copies land before the workgroup ends

  if (key < N) {
    store_transposed_acc<D>(dV + base + (int64_t)key * D, dv, g, 1.f);
    store_transposed_acc<D>(dK + base + (int64_t)key * D, dk, g, scale);
  }
}

// dQ for d = 64, run first: each workgroup also forms the per-row terms of
// its 256 query rows (those of bwd_preprocess_kernel: D from the saved O and
// dO, -LSE log2(e), and the two splits) and writes them for the dK/dV pass.
template <bool CAUSAL>
__global__ __launch_bounds__(kPPThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_dq_pp_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const __bf16* __restrict__ dO, const __bf16* __restrict__ O, const float* __restrict__ LSE,
    float* __restrict__ delta, float* __restrict__ nl2, u32x2* __restrict__ dsplit, u32x2* __restrict__ lsplit,
    __bf16* __restrict__ dQ, int N, int BH, int n_qtiles, int group, float scale, float scale_log2) {
  constexpr int D = 64;
  using T = TileLayout<D>;
  constexpr int NW = kPPWaves;
  constexpr int BQ = NW * 32;
  constexpr int kBuf = 2 * T::kBytes;
  __shared__ __attribute__((aligned(1024))) unsigned char sb0[kBuf];
  __shared__ __attribute__((aligned(1024))) unsigned char sb1[kBuf];
  __shared__ __attribute__((aligned(1024))) unsigned char sb2[kBuf];
  __shared__ __attribute__((aligned(1024))) unsigned char sb3[kBuf];

  int bh, qtile;
  head_tile(xcd_remap(blockIdx.x, BH * n_qtiles), n_qtiles, BH, group, bh, qtile);
  if (CAUSAL) qtile = n_qtiles - 1 - qtile;  // the last query tile sees the most keys
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool lead = wave < 4;
  const int g = lane >> 5, l32 = lane & 31;
  const int64_t base = (int64_t)bh * N * D;
  const int q0 = qtile * BQ;
  // the lead and the trail wavefront of SIMD s (w = s and w = s + 4) own row
  // blocks s and 7 - s, so on a causal diagonal every SIMD has the same work
  const int qw0 = q0 + 32 * (wave < 4 ? wave : 11 - wave);
  const int qr = qw0 + l32;

  const TileCopyBuf<D, NW> cp(wave, lane);
  const TileOffsets<D> of(lane);
  auto issue_tile = [&](int j, unsigned char* buf) __attribute__((always_inline)) {
    cp.issue(K + base, N, j * kT, buf);
    cp.issue(V + base, N, j * kT, buf + T::kBytes);
  };
  constexpr int kCopies = 2 * TileCopyBuf<D, NW>::kPerWave;
  auto wait_copies = [&](bool one_after) __attribute__((always_inline)) {
    if (one_after) wait_vm_at_most<kCopies>(); else wait_vm_at_most<0>();
  };

  const int kend = CAUSAL ? min(N, q0 + BQ) : N;
  const int ntiles = (kend + kT - 1) / kT;

  // The rows of this wavefront first (Q, dO, O, LSE), then tile 0: loads
  // complete in issue order, so the row terms wait for the rows only.
  bf16x8 qB[D / 16], doB[D / 16];
  u32x4 orow[D / 16];
  const int64_t row = (int64_t)bh * N + qr;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    qB[ks] = qr < N ? *reinterpret_cast<const bf16x8*>(Q + base + (int64_t)qr * D + 16 * ks + 8 * g) : bf16x8{};
    doB[ks] = qr < N ? *reinterpret_cast<const bf16x8*>(dO + base + (int64_t)qr * D + 16 * ks + 8 * g) : bf16x8{};
    orow[ks] = qr < N ? *reinterpret_cast<const u32x4*>(O + base + (int64_t)qr * D + 16 * ks + 8 * g) : u32x4{};
  }
  const float lse = LSE[(int64_t)bh * N + min(qr, N - 1)];  // unconditional: no branch to wait in
  issue_tile(0, sb0);
  __builtin_amdgcn_sched_barrier(0);  // tile 0 goes out before the wait for the rows
  // the row's terms: D = rowsum(dO o O) over the lane's 32 dims and its
  // partner's (lane ^ 32), -LSE log2(e), and the splits of -D and of
  // -LSE log2(e) / (scale log2(e))
  float dpart = 0.f;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    const u32x4 o = orow[ks];
    const u32x4 d = bitcast<u32x4>(doB[ks]);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      dpart = fmaf(bf16lo_to_f32(o[w]), bf16lo_to_f32(d[w]), dpart);
      dpart = fmaf(bf16hi_to_f32(o[w]), bf16hi_to_f32(d[w]), dpart);
    }
  }
  const float drow = dpart + shfl_xor_f32(dpart, 32);
  const float nlse2 = qr < N ? -lse * kLog2e : kNegInf;
  const u32x2 dwq = qr < N ? split3_bf16(-drow) : u32x2{0u, 0u};
  if (qr < N && g == 0) {
    delta[row] = drow;
    nl2[row] = nlse2;
    dsplit[row] = dwq;
    lsplit[row] = split3_bf16(nlse2 / scale_log2);
  }
  // dP^T - D starts from -D: the lane's query is the accumulator's column,
  // so all 16 of its elements start at the same value
  f32x16 negd;
#pragma unroll
  for (int i = 0; i < 16; ++i) negd[i] = -drow;
  f32x16 dq[D / 32];
#pragma unroll
  for (int mt = 0; mt < D / 32; ++mt) dq[mt] = f32x16{};
  f32x16 sacc, dpacc;             // S^T and dP^T - D of the current half
  bf16x8 sbf[2];                  // dS^T of the previous half, bf16
  bf16x8 rk[D / 16], rv[D / 16];  // K and V rows of the next half

  auto read_rows = [&](const int KH, const unsigned char* buf) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      rk[ks] = of.row(buf, ks, KH);
      rv[ks] = of.row(buf + T::kBytes, ks, KH);
    }
  };

  // M: S^T = K Q^T and dP^T - D of the current half, then dQ^T += K^T dS^T
  // of the previous half (tile at bprev, half 1 - KH).
  auto mph = [&](const int KH, const unsigned char* bprev, const bool do_acc, const bool do_scores)
      __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(1);
    const int KP = 1 - KH;
    bf16x8 tk[2][D / 32];
    if (do_acc) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int mt = 0; mt < D / 32; ++mt) tk[tt][mt] = of.tr(bprev, 2 * KP + tt, mt);
    }
    if (do_scores) {
      sacc = mfma32x32x16(rk[0], qB[0], f32x16{});
      dpacc = mfma32x32x16(rv[0], doB[0], negd);
#pragma unroll
      for (int ks = 1; ks < D / 16; ++ks) {
        sacc = mfma32x32x16(rk[ks], qB[ks], sacc);
        dpacc = mfma32x32x16(rv[ks], doB[ks], dpacc);
      }
    }
    if (do_acc) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int mt = 0; mt < D / 32; ++mt) dq[mt] = mfma32x32x16(tk[tt][mt], sbf[tt], dq[mt]);
    }
    if (do_acc && do_scores) {
      __builtin_amdgcn_sched_group_barrier(0x0100, 4 * (D / 32), 0);
      __builtin_amdgcn_sched_group_barrier(0x0008, 2 * (D / 16) + 2 * (D / 32), 0);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // V: dS^T = P^T o (dP^T - D) for the keys ka .. ka+31, packed to bf16; the
  // rows of the next half are read meanwhile.
  auto vph = [&](int ka, const bool next, const int NKH, const unsigned char* bnext)
      __attribute__((always_inline)) {
    if (next) read_rows(NKH, bnext);
    if ((ka + 31 >= N) || (CAUSAL && ka + 31 > qw0)) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kk = ka + acc_row(i, g);
        if (kk >= N || (CAUSAL && kk > qr)) sacc[i] = kNegInf;
      }
    }
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      float y[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int i = 8 * tt + e;
        y[e] = fast_exp2(fmaf(sacc[i], scale_log2, nlse2)) * dpacc[i];
      }
      sbf[tt] = pack_bf16x8(y);
    }
    asm volatile("" : "+v"(sbf[0]), "+v"(sbf[1]));
  };

  // tile 0 before the first barrier; tiles 1 and 2 go out after the first
  // products (a copy in flight there makes the compiler wait for every load)
  wait_vm_at_most<0>();
  lds_barrier();
  if (!lead) lds_barrier();
  read_rows(0, sb0);
  mph(0, sb0, false, true);
  // tiles past the last are empty copies into ring slots no step reads,
  // so the copies and the waits need no branches
  issue_tile(1, sb1);
  issue_tile(2, sb2);
  lds_barrier();
  vph(0, true, 1, sb0);
  wait_copies(true);
  lds_barrier();
  mph(1, sb0, true, true);
  lds_barrier();
  vph(32, ntiles > 1, 0, sb1);
  lds_barrier();
  auto step = [&](int s, const unsigned char* cur, const unsigned char* prev, const unsigned char* nxt1,
                  unsigned char* nxt2) __attribute__((always_inline)) {
    issue_tile(s + 2, nxt2);
    mph(0, prev, true, true);
    lds_barrier();
    vph(s * kT, true, 1, cur);
    wait_copies(true);
    lds_barrier();
    mph(1, cur, true, true);
    lds_barrier();
    vph(s * kT + 32, s + 1 < ntiles, 0, nxt1);
    lds_barrier();
  };
  // Causal: key tiles past the last one with a key visible to this
  // wavefront's rows are masked out for all of them; the wavefront stops
  // computing after that tile (nfull) and only copies and keeps the
  // workgroup's barrier count in the remaining steps.
  const int nfull = CAUSAL ? min(ntiles, (qw0 + 31) / kT + 1) : ntiles;
  for (int s = 1; s < nfull; s += 4) {
    step(s, sb1, sb0, sb2, sb3);
    if (s + 1 < nfull) step(s + 1, sb2, sb1, sb3, sb0);
    if (s + 2 < nfull) step(s + 2, sb3, sb2, sb0, sb1);
    if (s + 3 < nfull) step(s + 3, sb0, sb3, sb1, sb2);
  }
  auto slot = [&](int t) __attribute__((always_inline)) -> unsigned char* {
    t &= 3;
    return t == 0 ? sb0 : t == 1 ? sb1 : t == 2 ? sb2 : sb3;
  };
  // contraction of the last half of tile nfull - 1 (its ring slot is
  // overwritten only by tile nfull + 3, issued at the second step below)
  if (CAUSAL && nfull < ntiles) {
    for (int s = nfull; s < ntiles; ++s) {
      issue_tile(s + 2, slot(s + 2));
      if (s == nfull) mph(0, slot(nfull - 1), true, false);
      lds_barrier();
      wait_copies(true);
      lds_barrier();
      lds_barrier();
      lds_barrier();
    }
  } else {
    mph(0, slot(ntiles - 1), true, false);
  }
  if (lead) lds_barrier();
  wait_vm_at_most<0>();  // the last (empty) copies land before the workgroup ends

  if (qr < N) store_transposed_acc<D>(dQ + base + (int64_t)qr * D, dq, g, scale);
}

// fp32 zero fill (the atomic dQ accumulator; a kernel rather than a memset,
// so that the sequence can be captured in a graph)
__global__ __launch_bounds__(kThreads) void zero_f32x4_kernel(f32x4* __restrict__ p, int64_t n4) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n4; i += (int64_t)gridDim.x * kThreads)
    p[i] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// dQ = scale * accumulator, rounded to bf16 (RNE)
__global__ __launch_bounds__(kThreads) void dq_convert_kernel(const f32x4* __restrict__ acc, u32x2* __restrict__ dq,
                                                              float scale, int64_t n4) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n4; i += (int64_t)gridDim.x * kThreads) {
    const f32x4 v = acc[i];
    dq[i] = u32x2{pack_bf16x2(v[0] * scale, v[1] * scale), pack_bf16x2(v[2] * scale, v[3] * scale)};
  }
}

unsigned stream_grid(int64_t n4) {
  const int64_t wg = (n4 + kThreads - 1) / kThreads;
  return (unsigned)(wg < 16384 ? (wg > 0 ? wg : 1) : 16384);
}

// Per-row terms in the workspace: delta [rows] f32 | nl2 [rows] f32 |
// dsplit [rows] x 8 bytes | lsplit [rows] x 8 bytes
struct RowTerms {
  float* nl2;
  u32x2* dsplit;
  u32x2* lsplit;
};

template <int D>
hipError_t run_preprocess(const BwdArgs& a, hipStream_t s, RowTerms& t) {
  const int64_t rows = (int64_t)a.B * a.H * a.N;
  t.nl2 = a.delta + rows;
  t.dsplit = reinterpret_cast<u32x2*>(a.delta + 2 * rows);
  t.lsplit = t.dsplit + rows;
  constexpr int rows_per_wg = kThreads / (D / 8);
  hipLaunchKernelGGL((bwd_preprocess_kernel<D>), dim3((unsigned)((rows + rows_per_wg - 1) / rows_per_wg)),
                     dim3(kThreads), 0, s, static_cast<const __bf16*>(a.o), static_cast<const __bf16*>(a.dO),
                     a.lse, a.delta, t.nl2, t.dsplit, t.lsplit, a.scale * kLog2e, rows);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t run_bwd(const BwdArgs& a, hipStream_t s) {
  const int BH = a.B * a.H;
  const float scale_log2 = a.scale * kLog2e;
  const int group = BH >= kNumXcd ? BH / kNumXcd : 1;
  hipError_t e;
  if constexpr (D == 64) {
    // dQ first: it also writes the per-row terms that dK/dV reads
    const int64_t rows = (int64_t)BH * a.N;
    float* nl2 = a.delta + rows;
    u32x2* dsplit = reinterpret_cast<u32x2*>(a.delta + 2 * rows);
    u32x2* lsplit = dsplit + rows;
    const int n_qt = (a.N + kPPWaves * 32 - 1) / (kPPWaves * 32);
    hipLaunchKernelGGL((bwd_dq_pp_kernel<CAUSAL>), dim3(n_qt * BH), dim3(kPPThreads), 0, s,
                       static_cast<const __bf16*>(a.q), static_cast<const __bf16*>(a.k),
                       static_cast<const __bf16*>(a.v), static_cast<const __bf16*>(a.dO),
                       static_cast<const __bf16*>(a.o), a.lse, a.delta, nl2, dsplit, lsplit,
                       static_cast<__bf16*>(a.dq), a.N, BH, n_qt, group, a.scale, scale_log2);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int n_kt = (a.N + kPPWaves * 32 - 1) / (kPPWaves * 32);
    hipLaunchKernelGGL((bwd_dkdv_pp_kernel<CAUSAL>), dim3(n_kt * BH), dim3(kPPThreads), 0, s,
                       static_cast<const __bf16*>(a.q), static_cast<const __bf16*>(a.k),
                       static_cast<const __bf16*>(a.v), static_cast<const __bf16*>(a.dO), lsplit, dsplit,
                       static_cast<__bf16*>(a.dk), static_cast<__bf16*>(a.dv), a.N, BH, n_kt, group, a.scale,
                       scale_log2);
    return hipGetLastError();
  }
  RowTerms rt;
  e = run_preprocess<D>(a, s, rt);
  if (e != hipSuccess) return e;
  float* nl2 = rt.nl2;
  u32x2* dsplit = rt.dsplit;
  const int n_kt = (a.N + kWaves * 32 - 1) / (kWaves * 32);
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), dim3(n_kt * BH), dim3(kThreads), 0, s,
                     static_cast<const __bf16*>(a.q), static_cast<const __bf16*>(a.k),
                     static_cast<const __bf16*>(a.v), static_cast<const __bf16*>(a.dO), nl2, dsplit,
                     static_cast<__bf16*>(a.dk), static_cast<__bf16*>(a.dv), nullptr, a.N, BH, n_kt, group,
                     a.scale, scale_log2);
  e = hipGetLastError();
  if (e != hipSuccess) return e;

  const int n_qt = (a.N + kWaves * 32 - 1) / (kWaves * 32);
  hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL>), dim3(n_qt * BH), dim3(kThreads), 0, s,
                     static_cast<const __bf16*>(a.q), static_cast<const __bf16*>(a.k),
                     static_cast<const __bf16*>(a.v), static_cast<const __bf16*>(a.dO), nl2, dsplit,
                     static_cast<__bf16*>(a.dq), a.N, BH, n_qt, group, a.scale, scale_log2);
  return hipGetLastError();
}

// The atomic-dQ variant: preprocess, zero the fp32 accumulator, dK/dV with
// the dQ atomics, scale the accumulator into dQ.
template <int D, bool CAUSAL>
hipError_t run_bwd_atomic(const BwdArgs& a, hipStream_t s) {
  const int BH = a.B * a.H;
  const int64_t n4 = (int64_t)BH * a.N * D / 4;
  RowTerms rt;
  hipError_t e = run_preprocess<D>(a, s, rt);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(zero_f32x4_kernel, dim3(stream_grid(n4)), dim3(kThreads), 0, s,
                     reinterpret_cast<f32x4*>(a.dqacc), n4);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int group = BH >= kNumXcd ? BH / kNumXcd : 1;
  const int n_kt = (a.N + kWaves * 32 - 1) / (kWaves * 32);
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL, true>), dim3(n_kt * BH), dim3(kThreads), 0, s,
                     static_cast<const __bf16*>(a.q), static_cast<const __bf16*>(a.k),
                     static_cast<const __bf16*>(a.v), static_cast<const __bf16*>(a.dO), rt.nl2, rt.dsplit,
                     static_cast<__bf16*>(a.dk), static_cast<__bf16*>(a.dv), a.dqacc, a.N, BH, n_kt, group,
                     a.scale, a.scale * kLog2e);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(dq_convert_kernel, dim3(stream_grid(n4)), dim3(kThreads), 0, s,
                     reinterpret_cast<const f32x4*>(a.dqacc), static_cast<u32x2*>(a.dq), a.scale, n4);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_atomic_bf16(const BwdArgs& a, hipStream_t s) {
  if (a.d == 64) return a.causal ? run_bwd_atomic<64, true>(a, s) : run_bwd_atomic<64, false>(a, s);
  return a.causal ? run_bwd_atomic<128, true>(a, s) : run_bwd_atomic<128, false>(a, s);
}

hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t s) {
  if (a.d == 64) return a.causal ? run_bwd<64, true>(a, s) : run_bwd<64, false>(a, s);
  return a.causal ? run_bwd<128, true>(a, s) : run_bwd<128, false>(a, s);
}

}  // namespace attn
