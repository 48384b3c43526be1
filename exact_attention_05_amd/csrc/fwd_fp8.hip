// FP8 (E4M3) attention forward and block quantisation for gfx950
// ("8. FlashAttention 实战", triton-tutorial.pages.dev, section 8.9).
//
// Storage: Q, K, V in E4M3 with one fp32 scale per block of rows, the page's
// max|x| / 448 (section 8.9.4): Q per 32 rows (BLOCK_M), K and V per 64
// (BLOCK_N).  The quantiser below writes both.
//
// Forward (d = 64), the method of section 8.9.3 and the listing of section
// 8.9.6 with BLOCK_M = 32 query rows (one wavefront) and BLOCK_N = 64 keys
// (one K/V tile).  Eight wavefronts of 32 query rows per workgroup, two
// workgroups per CU (four wavefronts per SIMD), the wavefronts of a workgroup
// in two groups one phase apart as in the bf16 d = 64 kernel, 64-key tiles
// copied HBM -> LDS ahead of use; causal: as there, a wavefront stops after
// its last key tile with a visible key and SIMD s holds row blocks s and 7 - s.
// Per tile j and wavefront:
//   S^T = K8 Q8^T     two FP8 MFMAs (keys 0-31, 32-63), the whole d = 64
//                     reduction in one instruction each;
//   u = S sq sk_j scale log2(e)          (scores in base-2 units; masked)
//   m_new = max(m, rowmax u), alpha = 2^(m - m_new)       (per query row)
//   e = max over the block's rows of (rowmax u - m_new)    (wave-wide):
//                     the block's largest p = 2^(u - m_new) is 2^e, so
//                     scale_p = 2^e / 448 and p / scale_p = 2^(u - m_new - e) 448
//   P8 = e4m3(p / scale_p)   (the probabilities requantised to FP8)
//   l = alpha l + 2^e / 448 * sum(p / scale_p)   (p unrounded, as the page's l)
//   T = V8^T P8^T     two FP8 MFMAs in the next matrix phase, and there
//   U = alpha U + (scale_p sv_j) T            (the block's product scaled by
//                     its own scales; the listing scales the whole accumulator)
//                     before the next tile's score products, so T and S are
//                     never live together (no register spills at 128 VGPRs)
// and at the end O = U / l, LSE = (m + log2 l) ln 2.  The kernel keeps U and l
// multiplied by 2^(m - mref), mref a per-row reference (the first visible
// block's m, moved up when m passes it by 64): alpha U then needs no
// multiply, a block's T goes in with the factor scale_p sv_j 2^(m_new - mref),
// the factor cancels in O, and LSE = (mref + log2 l) ln 2.  Rows past N do not take
// part in the block's max.  P8 goes from the score accumulator straight into
// the B operand (a lane holds 32 keys of its query); the V^T operand is read
// with transposing 8-bit LDS reads whose source rows follow the same key
// order.
#include "common.h"
#include "launch.h"

namespace attn {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

constexpr int kFp8Bc = 64;        // keys per tile (BLOCK_N)
constexpr int kFp8Row = 64;       // bytes per row (d = 64, one byte each)
constexpr int kFp8Tile = 64 * 64; // bytes per K or V tile
constexpr float kP8Max = 448.f;   // largest finite E4M3 value
constexpr float kLog2P8Max = 8.807354922057604f;  // log2(448)
constexpr int kE8One = 127;       // E8M0 encoding of 1.0

__device__ __forceinline__ f32x16 mfma_fp8(const i32x8& a, const i32x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, kE8One, 0, kE8One);
}

// Transposing LDS read of 8-bit values (ds_read_b64_tr_b8).  Within every
// group of 16 lanes each lane names 8 bytes; lane i of the group receives, as
// its byte q, byte (i % 8) of the 8 bytes named by lane 2q + i / 8.
__device__ __forceinline__ i32x2 lds_read_tr8(const void* lds_addr) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2*)lds_addr);
}

// FP8 tile: 64 rows x 64 bytes, row k at byte 64k, its 16-byte chunk c stored
// at chunk c ^ ((k >> 2) & 3).  Both operand reads then touch every LDS bank
// once per pass: 16 consecutive rows x one chunk (ds_read_b128), and 8 rows
// {k0..k0+3, k0+8..k0+11} x 4 chunk-halves (ds_read_b64_tr_b8, 32 lanes).
__device__ __forceinline__ int fp8_off(int k, int c) { return 64 * k + 16 * (c ^ ((k >> 2) & 3)); }

// Key of byte J of a lane in half h of the P8 operand: the score
// accumulator's row order (block J / 16, accumulator index J % 16).
__device__ __forceinline__ constexpr int pkey(int h, int J) { return 32 * (J >> 4) + acc_row(J & 15, h); }

// v_max_f32 / v_max3_f32 as plain instructions.  The compiler puts a
// canonicalising v_max_f32 x, x, x in front of every fmaxf operand it cannot
// prove canonical (MFMA results, lane reads), which doubles the per-tile row
// max.  The operands here are never signalling NaNs; on quiet NaNs and
// infinities the instructions give what fmaxf gives.
__device__ __forceinline__ float vmax(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float vmax3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// v_permlane32_swap of x with itself: the first result holds x of lanes
// 0-31 in both halves of the wave, the second x of lanes 32-63; a symmetric
// combination of the two is the lane pair's (l, l ^ 32) value in every lane.
__device__ __forceinline__ float max_of_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_of_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Max of `x` over lanes 0-31 (lanes 32-63 hold the same values), wave-uniform.
__device__ __forceinline__ float max_over_32_lanes(float x) {
  // every source lane of these patterns lies in the destination's row
#define ATTN_DPP(v, ctrl) __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), ctrl, 0xF, 0xF, true))
  x = vmax(x, ATTN_DPP(x, 0xB1));   // quad_perm 1,0,3,2
  x = vmax(x, ATTN_DPP(x, 0x4E));   // quad_perm 2,3,0,1
  x = vmax(x, ATTN_DPP(x, 0x141));  // row_half_mirror
  x = vmax(x, ATTN_DPP(x, 0x140));  // row_mirror
#undef ATTN_DPP
  return fmaxf(__uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(x), 0)),
               __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(x), 16)));
}

// ---------------------------------------------------------------------------
// Forward kernel, d = 64.  Work ids, eight wavefronts (256 query rows) per
// workgroup, two workgroups per CU, ring of five tiles, phase structure and
// barriers as fwd_pp4_kernel.  Every wavefront copies 1 KB of the K tile or
// the V tile.
// ---------------------------------------------------------------------------
template <bool CAUSAL>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4, 4))) void fwd_fp8_kernel(
    const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K, const uint8_t* __restrict__ V,
    const float* __restrict__ QS, const float* __restrict__ KS, const float* __restrict__ VS,
    __bf16* __restrict__ O, float* __restrict__ LSE, int N, int n_qtiles, int total_wg, float scale_log2) {
  constexpr int D = 64;
  constexpr int NW = 8;
  constexpr int BR = NW * 32;
  constexpr int TB = 2 * kFp8Tile;  // K | V
  __shared__ __attribute__((aligned(1024))) unsigned char sb0[TB];
  __shared__ __attribute__((aligned(1024))) unsigned char sb1[TB];
  __shared__ __attribute__((aligned(1024))) unsigned char sb2[TB];
  __shared__ __attribute__((aligned(1024))) unsigned char sb3[TB];
  __shared__ __attribute__((aligned(1024))) unsigned char sb4[TB];

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
  const int qw0 = q0 + 32 * (wave < NW / 2 ? wave : 3 * NW / 2 - 1 - wave);
  const int qr = qw0 + l32;
  const int kend = CAUSAL ? min(N, q0 + BR) : N;
  const int ntiles = (kend + kFp8Bc - 1) / kFp8Bc;
  const int nkb = (N + kFp8Bc - 1) / kFp8Bc;
  const float* ksh = KS + (int64_t)bh * nkb;
  const float* vsh = VS + (int64_t)bh * nkb;

  // copy geometry: waves 0-3 fill the K tile, 4-7 the V tile, 1 KB each;
  // lane l fills physical chunk l % 4 of row 16 (wave % 4) + l / 4.
  const uint8_t* csrc = (wave < 4 ? K : V) + base;  // wave-uniform
  const int crow = 16 * (wave & 3) + (lane >> 2);
  const int cvoff = crow * kFp8Row + 16 * ((lane & 3) ^ ((crow >> 2) & 3));
  const int cdst = (wave < 4 ? 0 : kFp8Tile) + 1024 * (wave & 3);
  auto issue_tile = [&](int j, unsigned char* buf) __attribute__((always_inline)) {
    // one buffer descriptor per tile: rows past N read zeros (masked later)
    const int r0 = j * kFp8Bc;
    buffer_to_lds16(csrc + (int64_t)r0 * kFp8Row, (uint32_t)(N - r0) * kFp8Row, cvoff, buf + cdst);
  };

  // Q row of this lane: bytes 32g .. 32g+31 (the B operand's reduction half g)
  i32x8 qB = {};
  if (qr < N) {
    const u32x4* qp = reinterpret_cast<const u32x4*>(Q + base + (int64_t)qr * kFp8Row + 32 * g);
    const u32x4 a = qp[0], b = qp[1];
    qB = i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
  }
  issue_tile(0, sb0);
  // the wavefront's 32 rows are one Q scale block
  const float cq = scale_log2 * QS[(int64_t)bh * ((N + 31) / 32) + min(qw0, N - 1) / 32];

  // Per-lane LDS offsets.  K rows (S operand): chunks 2g and 2g+1 of row
  // l32; rows 32 further (the second key half) share the swizzle phase, +2048.
  const int koff0 = fp8_off(l32, 2 * g), koff1 = fp8_off(l32, 2 * g + 1);
  // Transposed V (O operand): the source lane of read t names key
  // pkey(G / 2, 8t + q) = 16t + kl and dims 32mt + 16(G % 2) + 8p; the key's
  // swizzle phase does not depend on t (+1024 per read), and d block mt = 1
  // flips bit 1 of the chunk (XOR 32).
  int voff0;
  {
    const int G = lane >> 4, s = lane & 15, qq = s >> 1, pp = s & 1;
    voff0 = fp8_off(pkey(G >> 1, qq), G & 1) + 8 * pp;
  }

  f32x16 oacc[2] = {f32x16{}, f32x16{}};
  f32x16 tacc[2];  // T = V8^T P8^T of the previous tile
  // U and l are kept multiplied by 2^(m - mref): a block's product then goes
  // in with one fma, and the factor cancels in O = U / l (LSE = mref + log2 l)
  float m = kNegInf, mref = kNegInf, lsum = 0.f;
  float f_prev = 0.f;  // the previous tile's scale_p sv 2^(m - mref) (per row)
  f32x16 sacc[2];
  i32x8 pb = {};  // P8 of the current tile, the B operand of T
  float ck = cq * ksh[0];

  // MFMA operands, all read from LDS at the top of the matrix phase so that
  // their latencies overlap (V^T of the previous tile, K of this one).
  i32x8 va[2], ka[2];
  auto read_k = [&](const unsigned char* kt) __attribute__((always_inline)) {
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const u32x4 a = *reinterpret_cast<const u32x4*>(kt + koff0 + 2048 * hb);
      const u32x4 b = *reinterpret_cast<const u32x4*>(kt + koff1 + 2048 * hb);
      ka[hb] = i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
    }
  };
  auto read_v = [&](const unsigned char* vt) __attribute__((always_inline)) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int vo = mt ? (voff0 ^ 32) : voff0;
      i32x2 r[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) r[t] = lds_read_tr8(vt + vo + 1024 * t);
      va[mt] = i32x8{r[0][0], r[0][1], r[1][0], r[1][1], r[2][0], r[2][1], r[3][0], r[3][1]};
    }
  };
  // U += f T for the previous tile's product (f carries the frame factor)
  auto accumulate = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[mt][i] = fmaf(tacc[mt][i], f_prev, oacc[mt][i]);
  };

  // M: T = V^T P8^T of the previous tile, added into U with that tile's
  // factor, then S^T of this one; the K operands are read after the
  // addition so that T and S are never live together.  `copy` runs after the
  // V operand reads: a tile copy issued before them makes the compiler wait
  // for it (it cannot always tell the buffers apart).
  auto mph = [&](const unsigned char* kt, const unsigned char* vt, const bool do_pv, const bool do_s,
                 auto&& copy) __attribute__((always_inline)) {
    if (do_pv) read_v(vt + kFp8Tile);
    copy();
    __builtin_amdgcn_s_setprio(1);
    if (do_pv) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) tacc[mt] = mfma_fp8(va[mt], pb, f32x16{});
      __builtin_amdgcn_sched_barrier(0);
      accumulate();
      asm volatile("" : "+v"(oacc[0]), "+v"(oacc[1])::"memory");
    }
    if (do_s) read_k(kt);
    if (do_s) {
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) sacc[hb] = mfma_fp8(ka[hb], qB, f32x16{});
    }
    // keep the products in this phase (the barrier after it orders memory only)
    if (do_s) asm volatile("" : "+v"(sacc[0]), "+v"(sacc[1]));
    __builtin_amdgcn_s_setprio(0);
  };
  auto mask_tile = [&](int j) __attribute__((always_inline)) {
    const int kb = j * kFp8Bc;
    if ((kb + kFp8Bc > N) || (CAUSAL && kb + kFp8Bc - 1 > qw0)) {
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kb + 32 * hb + acc_row(i, g);
          const bool vis = key < N && (!CAUSAL || key <= qr);
          if (!vis) sacc[hb][i] = kNegInf;
        }
    }
  };
  // V(j): the previous tile's product into U, then the online softmax of tile j.
  auto vph = [&](int j) __attribute__((always_inline)) {
    mask_tile(j);
    // row max of the raw scores (the block's scales are positive)
    float mx0 = kNegInf, mx1 = kNegInf;
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      mx0 = vmax3(mx0, sacc[0][i], sacc[1][i]);
      mx1 = vmax3(mx1, sacc[0][i + 1], sacc[1][i + 1]);
    }
    const float mx = max_of_halves(vmax(mx0, mx1));
    const float bm = mx * ck;  // the row's largest u in this block (-inf: none visible)
    const float m_new = vmax(m, bm);
    // the first visible block fixes the frame; a frame more than 2^64 below
    // the running max is moved up to it (rare: U and l are rescaled)
    if (__builtin_expect(__ballot(m_new - mref > 64.f) != 0, 0)) {
      const float r = m_new - mref > 64.f ? fast_exp2(mref - m_new) : 1.f;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) oacc[mt] *= r;
      lsum *= r;
      mref = m_new - mref > 64.f ? m_new : mref;
    }
    mref = mref == kNegInf ? m_new : mref;
    const float gf = m_new == kNegInf ? 0.f : fast_exp2(m_new - mref);
    // e = log2 of the block's largest p, over its rows below N
    const float e = max_over_32_lanes(qr < N ? bm - m_new : kNegInf);
    const float off = e == kNegInf ? 0.f : m_new + e - kLog2P8Max;
    float r4[4];
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      float x[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) x[q] = fast_exp2(fmaf(sacc[w >> 2][4 * (w & 3) + q], ck, -off));
      if ((w & 1) == 0) r4[w >> 1] = (x[0] + x[1]) + (x[2] + x[3]);
      else r4[w >> 1] += (x[0] + x[1]) + (x[2] + x[3]);
      // both halves of the word are written: the previous tile's codes (read
      // by the last matrix phase) only stand in for the old value
      const int pw = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], pb[w], false);
      pb[w] = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], pw, true);
    }
    const float rs = (r4[0] + r4[1]) + (r4[2] + r4[3]);
    const float sp = fast_exp2(e) * (1.f / kP8Max);  // scale_p (0 for an empty block)
    lsum = fmaf(rs, sp * gf, lsum);
    m = m_new;
    f_prev = sp * vsh[j] * gf;
    if (j + 1 < ntiles) ck = cq * ksh[j + 1];
    asm volatile("" : "+v"(pb));
  };

  // Q and tile 0 land before the first barrier; tiles 1-3 are issued after
  // the first products (a copy in flight there makes the compiler wait for
  // every load before them)
  wait_vm_at_most<0>();
  lds_barrier();
  if (!lead) lds_barrier();
  mph(sb0, sb0, false, true, []() __attribute__((always_inline)) {});
  if (ntiles > 1) issue_tile(1, sb1);
  if (ntiles > 2) issue_tile(2, sb2);
  if (ntiles > 3) issue_tile(3, sb3);
  if (ntiles > 3) wait_vm_at_most<2>(); else if (ntiles > 2) wait_vm_at_most<1>(); else wait_vm_at_most<0>();
  lds_barrier();
  vph(0);
  // Tile j at cur, j-1 at prev; tile j+3 goes to far (the slot of j-2).
  auto step = [&](int j, const unsigned char* cur, const unsigned char* prev, unsigned char* far)
      __attribute__((always_inline)) {
    lds_barrier();
    mph(cur, prev, true, true, [&]() __attribute__((always_inline)) { if (j + 3 < ntiles) issue_tile(j + 3, far); });
    if (j + 3 < ntiles) wait_vm_at_most<2>(); else if (j + 2 < ntiles) wait_vm_at_most<1>(); else wait_vm_at_most<0>();
    lds_barrier();
    vph(j);
  };
  // Causal: key tiles past the last one with a key visible to this
  // wavefront's rows are masked out for all of them; the wavefront stops
  // computing after that tile (nfull) and only copies and keeps the
  // workgroup's barrier count in the remaining steps.
  const int nfull = CAUSAL ? min(ntiles, (qw0 + 31) / kFp8Bc + 1) : ntiles;
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
    // the P8 V product of tile nfull - 1 (its ring slot is overwritten only
    // by tile nfull + 4, issued at the second step below)
    {
      const int j = nfull;
      lds_barrier();
      mph(slot(j), slot(j - 1), true, false, [&]() __attribute__((always_inline)) {
        if (j + 3 < ntiles) issue_tile(j + 3, slot(j + 3));
      });
      if (j + 3 < ntiles) wait_vm_at_most<2>(); else if (j + 2 < ntiles) wait_vm_at_most<1>(); else wait_vm_at_most<0>();
      lds_barrier();
    }
    for (int j = nfull + 1; j < ntiles; ++j) {
      lds_barrier();
      if (j + 3 < ntiles) issue_tile(j + 3, slot(j + 3));
      if (j + 3 < ntiles) wait_vm_at_most<2>(); else if (j + 2 < ntiles) wait_vm_at_most<1>(); else wait_vm_at_most<0>();
      lds_barrier();
    }
    lds_barrier();
  } else {
    lds_barrier();
    mph(slot(ntiles - 1), slot(ntiles - 1), true, false, []() {});
  }
  if (lead) lds_barrier();

  const float lt = sum_of_halves(lsum);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (qr < N) {
    __bf16* Oh = O + base;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int d0 = 32 * mt + 8 * c + 4 * g;
        u32x2 w = {pack_bf16x2(oacc[mt][4 * c] * inv, oacc[mt][4 * c + 1] * inv),
                   pack_bf16x2(oacc[mt][4 * c + 2] * inv, oacc[mt][4 * c + 3] * inv)};
        *reinterpret_cast<u32x2*>(Oh + (int64_t)qr * D + d0) = w;
      }
    if (g == 0 && LSE != nullptr) LSE[(int64_t)bh * N + qr] = lt > 0.f ? (mref + fast_log2(lt)) * kLn2 : kNegInf;
  }
}

// ---------------------------------------------------------------------------
// Block quantisation ("8. FlashAttention 实战", section 8.9.4): one workgroup
// per block of rows of one (b, h).  Each thread holds 8 consecutive values of
// a row (D / 8 threads per row).  With signs, each row is first rotated,
// y = (x o signs) H / sqrt(D) (section 8.9.5; fast Walsh-Hadamard transform:
// three butterfly stages inside the thread, the rest across the row's lanes).
// Pass 1 takes max|y| over the block; the scale is max|y| / 448 (1 for an
// all-zero block), an IEEE fp32 division as in the page's tensor code; pass 2
// writes e4m3(clamp(y / scale, +-448)), y / scale again divided in fp32 and
// rounded to nearest even.  When the block spans at most NP passes of rows,
// its values stay in registers after one read (all loads issued before any
// is used); NP = 0 reads the block twice.
// ---------------------------------------------------------------------------
template <int D, bool ROT, int NP>
__global__ __launch_bounds__(256) void quant_fp8_kernel(const __bf16* __restrict__ X, const float* __restrict__ signs,
                                                        uint8_t* __restrict__ X8, float* __restrict__ scales,
                                                        int N, int block_rows, int nblk) {
  constexpr int TPR = D / 8;        // threads per row
  constexpr int RPP = 256 / TPR;    // rows per pass
  __shared__ float red[4];
  const int bh = blockIdx.x / nblk;
  const int b = blockIdx.x % nblk;
  const int r0 = b * block_rows;
  const int r1 = min(r0 + block_rows, N);
  const int tid = threadIdx.x;
  const int u = tid % TPR;          // dims 8u .. 8u+7
  const __bf16* Xh = X + (int64_t)bh * N * D;

  float sg[8];
  if constexpr (ROT) {
#pragma unroll
    for (int e = 0; e < 8; ++e) sg[e] = signs[8 * u + e];
  }
  auto load_row = [&](int r, float (&y)[8]) __attribute__((always_inline)) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(Xh + (int64_t)r * D + 8 * u);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      y[2 * e] = bf16lo_to_f32(w[e]);
      y[2 * e + 1] = bf16hi_to_f32(w[e]);
    }
    if constexpr (ROT) {
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] *= sg[e];
#pragma unroll
      for (int hb = 1; hb < 8; hb <<= 1)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if ((e & hb) == 0) {
            const float a = y[e], c = y[e + hb];
            y[e] = a + c;
            y[e + hb] = a - c;
          }
#pragma unroll
      for (int lb = 1; lb < TPR; lb <<= 1) {
        const bool hi = (u & lb) != 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float o = shfl_xor_f32(y[e], lb);
          y[e] = hi ? o - y[e] : y[e] + o;
        }
      }
      static_assert(D == 64, "rotation normalisation is exact only for d = 64");
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] *= 0.125f;  // 1 / sqrt(64)
    }
  };

  // Every thread runs the same number of passes (the rotation's shuffles need
  // all lanes of a row); rows past the block read row r0 and are discarded.
  const int npass = (r1 - r0 + RPP - 1) / RPP;

  // pass 1: max |y| over the block
  float amax = 0.f;
  float held[NP > 0 ? NP : 1][8];
  if constexpr (NP > 0) {
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int r = r0 + p * RPP + tid / TPR;
      if (p < npass) load_row(r < r1 ? r : r0, held[p]);
    }
#pragma unroll
    for (int p = 0; p < NP; ++p)
      if (p < npass && r0 + p * RPP + tid / TPR < r1) {
#pragma unroll
        for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(held[p][e]));
      }
  } else {
    for (int p = 0; p < npass; ++p) {
      const int r = r0 + p * RPP + tid / TPR;
      float y[8];
      const bool ok = r < r1;
      load_row(ok ? r : r0, y);
      if (ok) {
#pragma unroll
        for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(y[e]));
      }
    }
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) amax = fmaxf(amax, shfl_xor_f32(amax, m));
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));

  const float scale = amax > 0.f ? __fdiv_rn(amax, kP8Max) : 1.f;
  if (tid == 0) scales[(int64_t)bh * nblk + b] = scale;

  // pass 2: codes
  uint8_t* X8h = X8 + (int64_t)bh * N * D;
  auto store_row = [&](int r, const float (&y)[8]) __attribute__((always_inline)) {
    uint32_t w[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float z[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) z[e] = fminf(fmaxf(__fdiv_rn(y[4 * h + e], scale), -kP8Max), kP8Max);
      int pw = __builtin_amdgcn_cvt_pk_fp8_f32(z[0], z[1], 0, false);
      w[h] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(z[2], z[3], pw, true);
    }
    *reinterpret_cast<u32x2*>(X8h + (int64_t)r * D + 8 * u) = u32x2{w[0], w[1]};
  };
  if constexpr (NP > 0) {
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int r = r0 + p * RPP + tid / TPR;
      if (p < npass && r < r1) store_row(r, held[p]);
    }
  } else {
    for (int p = 0; p < npass; ++p) {
      const int r = r0 + p * RPP + tid / TPR;
      float y[8];
      const bool ok = r < r1;
      load_row(ok ? r : r0, y);
      if (ok) store_row(r, y);
    }
  }
}

template <bool CAUSAL>
hipError_t run_fp8(const Fp8FwdArgs& a, hipStream_t s) {
  constexpr int BR = 8 * 32;
  const int n_qtiles = (a.N + BR - 1) / BR;
  const int total = n_qtiles * a.B * a.H;
  hipLaunchKernelGGL((fwd_fp8_kernel<CAUSAL>), dim3(total), dim3(512), 0, s, static_cast<const uint8_t*>(a.q),
                     static_cast<const uint8_t*>(a.k), static_cast<const uint8_t*>(a.v), a.q_scale, a.k_scale,
                     a.v_scale, static_cast<__bf16*>(a.o), a.lse, a.N, n_qtiles, total, a.scale * kLog2e);
  return hipGetLastError();
}

template <int D, bool ROT, int NP>
hipError_t run_quant_np(const QuantArgs& a, hipStream_t s) {
  const int nblk = (a.N + a.block_rows - 1) / a.block_rows;
  const int64_t grid = (int64_t)a.B * a.H * nblk;
  hipLaunchKernelGGL((quant_fp8_kernel<D, ROT, NP>), dim3((unsigned)grid), dim3(256), 0, s,
                     static_cast<const __bf16*>(a.x), a.signs, static_cast<uint8_t*>(a.x8), a.scales, a.N,
                     a.block_rows, nblk);
  return hipGetLastError();
}

// passes of 256 / (D / 8) rows that one block needs: held in registers up to 4
template <int D, bool ROT>
hipError_t run_quant(const QuantArgs& a, hipStream_t s) {
  constexpr int RPP = 256 / (D / 8);
  const int rows = a.block_rows < a.N ? a.block_rows : a.N;
  const int np = (rows + RPP - 1) / RPP;
  if (np <= 1) return run_quant_np<D, ROT, 1>(a, s);
  if (np <= 2) return run_quant_np<D, ROT, 2>(a, s);
  if (np <= 4) return run_quant_np<D, ROT, 4>(a, s);
  return run_quant_np<D, ROT, 0>(a, s);
}

}  // namespace

hipError_t launch_fwd_fp8(const Fp8FwdArgs& a, hipStream_t s) {
  return a.causal ? run_fp8<true>(a, s) : run_fp8<false>(a, s);
}

hipError_t launch_quantize_fp8(const QuantArgs& a, hipStream_t s) {
  if (a.signs != nullptr) return run_quant<64, true>(a, s);
  return a.d == 64 ? run_quant<64, false>(a, s) : run_quant<128, false>(a, s);
}

}  // namespace attn
