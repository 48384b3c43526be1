// Device helpers shared by the gfx950 attention kernels: vector types, MFMA
// wrappers, bf16 conversion, exp2, LDS copies and reads, the LDS tile layout,
// the launch-order remap for the 8 XCDs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

// ---------------------------------------------------------------------------
// MFMA: D(32x32, fp32) += A(32xK) * B(Kx32).
// Operand layout (wave64): lane l supplies row/column (l % 32) of A/B and the
// K-slice selected by (l / 32); the accumulator element i of lane l holds
// row 8*(i/4) + 4*(l/32) + (i%4), column l % 32.
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x16 mfma32x32x16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma32x32x2f32(float a, float b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Row index (within a 32-row accumulator tile) of element i in lane group g.
__device__ __forceinline__ constexpr int acc_row(int i, int g) { return 8 * (i >> 2) + 4 * g + (i & 3); }

// ---------------------------------------------------------------------------
// bf16 <-> fp32
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Reinterpretation through memcpy: __builtin_bit_cast of a vector ELEMENT
// (e.g. bit_cast<bf16x2>(u32x4_value[w])) is miscompiled by this hipcc (every
// element reads element 0), so all reinterpretations go through these.
template <typename To, typename From>
__device__ __forceinline__ To bitcast(const From& f) {
  static_assert(sizeof(To) == sizeof(From), "size mismatch");
  To t;
  __builtin_memcpy(&t, &f, sizeof(To));
  return t;
}

__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t w) { return bitcast<bf16x2>(w); }

// Two fp32 -> packed bf16 pair (round to nearest even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return bitcast<uint32_t>(v);
}

__device__ __forceinline__ bf16x8 pack_bf16x8(const float* x) {
  u32x4 u;
  u[0] = pack_bf16x2(x[0], x[1]);
  u[1] = pack_bf16x2(x[2], x[3]);
  u[2] = pack_bf16x2(x[4], x[5]);
  u[3] = pack_bf16x2(x[6], x[7]);
  return bitcast<bf16x8>(u);
}

// Hardware base-2 exponential (v_exp_f32); exp2(-inf) = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// log2 of a positive normal float (v_log_f32).
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ float shfl_xor_f32(float v, int mask) { return __shfl_xor(v, mask, 64); }

// ---------------------------------------------------------------------------
// LDS access helpers (gfx950)
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void;
typedef short i16x4 __attribute__((ext_vector_type(4)));

// Direct HBM -> LDS copy of 16 bytes per lane: lane l's bytes land at
// lds_base + 16 * l (lds_base must be the same for the whole wavefront).
__device__ __forceinline__ void global_to_lds16(const void* gptr, void* lds_base) {
  __builtin_amdgcn_global_load_lds(gptr, (lds_void*)lds_base, 16, 0, 0);
}

// Direct HBM -> LDS copy of 4 bytes per lane: lane l's word lands at
// lds_base + 4 * l.
__device__ __forceinline__ void global_to_lds4(const void* gptr, void* lds_base) {
  __builtin_amdgcn_global_load_lds(gptr, (lds_void*)lds_base, 4, 0, 0);
}

// Transposing LDS read (ds_read_b64_tr_b16).  Within every group of 16 lanes,
// each lane names 8 bytes (4 consecutive 16-bit values); lane i of the group
// receives, as its element j, element (i % 4) of the 8 bytes named by lane
// 4 * j + i / 4 of the group.
__device__ __forceinline__ u32x2 lds_read_tr16(const void* lds_addr) {
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)lds_addr);
  return bitcast<u32x2>(v);
}

// Wait until every memory operation this wavefront issued has completed
// (including direct-to-LDS copies).
__device__ __forceinline__ void wait_all_memory() { __builtin_amdgcn_s_waitcnt(0); }

// Workgroup barrier for LDS hand-offs that must not wait on the wavefront's
// outstanding global->LDS copies (__syncthreads() would, through its
// workgroup-scope fences).  Callers make their own copies complete with
// wait_vm_at_most before it.  LDS reads issued before it have returned
// (lgkmcnt(0)), and the asm clobbers keep the compiler from moving memory
// accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0) only
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Wait until at most N vector-memory operations of this wavefront are
// outstanding (s_waitcnt vmcnt(N); LDS and export counters not waited on).
template <int N>
__device__ __forceinline__ void wait_vm_at_most() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// ---------------------------------------------------------------------------
// Tile layout in LDS.  A tile of 64 rows (keys or queries) x D bf16 is stored
// row-major (row k, dims d) as a sequence of 256-byte lines -- 64 banks of 4
// bytes --
// and the 16-byte chunks inside a line are XOR-swizzled by a function of the
// line index.  ds_read_b128 is served 16 lanes (256 bytes) per pass and
// ds_read_b64_tr_b16 32 lanes per pass; the swizzle makes every pass touch
// each of the 64 banks once:
//   * row-operand reads: 16 consecutive rows, one chunk each -- the swizzle
//     is a permutation of the chunk index over every 8 (d = 64) or 16
//     (d = 128) aligned lines;
//   * transposing reads: 4 consecutive rows x 4 aligned chunks -- the lines
//     holding those rows XOR the 4-chunk block into distinct quarters (the
//     low line bits drive the high swizzle bits).
// d = 64: row k lives in line k/2, chunks 8*(k%2) .. 8*(k%2)+7.
// d = 128: row k is line k.
template <int D>
struct TileLayout {
  static constexpr int kLines = D / 2;        // 256-byte lines per tile
  static constexpr int kBytes = kLines * 256;  // = 64 * D * 2
  __device__ static __forceinline__ int swz(int line) {
    if constexpr (D == 64) return ((line & 1) << 2) | ((line >> 1) & 3);
    else return ((line & 3) << 2) | ((line >> 2) & 3);
  }
  // byte offset of logical 16-byte chunk c of row k
  __device__ static __forceinline__ int offset(int k, int c) {
    const int lin = k * (D * 2) + 16 * c;  // unswizzled byte offset
    const int line = lin >> 8;
    const int chunk = (lin >> 4) & 15;
    return line * 256 + 16 * (chunk ^ swz(line));
  }
  // inverse: the (row, chunk) stored at physical chunk p of line `line`
  __device__ static __forceinline__ void at(int line, int p, int& k, int& c) {
    const int chunk = p ^ swz(line);
    const int lin = line * 256 + 16 * chunk;
    k = lin / (D * 2);
    c = (lin % (D * 2)) / 16;
  }
};

// ---------------------------------------------------------------------------
// Per-lane LDS offsets of the MFMA operands in a TileLayout tile:
//   row operand of ks-slice ks, rows 32h + l32: roff[ks] + h * kHalf;
//   transposing operand of 16-row slice t, dims 32mt..+31: toff[0/1][mt] + t * kTStep.
// ---------------------------------------------------------------------------
template <int D>
struct TileOffsets {
  using T = TileLayout<D>;
  static constexpr int kHalf = 32 * D * 2;   // 32 rows further: same swizzle phase
  static constexpr int kTStep = 16 * D * 2;  // 16 rows further
  int roff[D / 16];
  int toff[2][D / 32];
  __device__ __forceinline__ TileOffsets(int lane) {
    const int g = lane >> 5, l32 = lane & 31;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) roff[ks] = T::offset(l32, 2 * ks + g);
    const int sl = lane & 15, G = lane >> 4;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int mt = 0; mt < D / 32; ++mt) {
        const int row = 8 * h + 4 * (G >> 1) + (sl >> 2);
        const int dim = 32 * mt + 16 * (G & 1) + 4 * (sl & 3);
        toff[h][mt] = T::offset(row, dim >> 3) + 8 * ((dim >> 2) & 1);
      }
  }
  // transposed operand: 16 consecutive rows (slice t, in the accumulator's
  // row order) x 32 dims, as an MFMA A operand
  __device__ __forceinline__ bf16x8 tr(const unsigned char* tile, int t, int mt) const {
    const u32x2 lo = lds_read_tr16(tile + toff[0][mt] + t * kTStep);
    const u32x2 hi = lds_read_tr16(tile + toff[1][mt] + t * kTStep);
    const u32x4 w = {lo[0], lo[1], hi[0], hi[1]};
    return bitcast<bf16x8>(w);
  }
  __device__ __forceinline__ bf16x8 row(const unsigned char* tile, int ks, int h) const {
    return *reinterpret_cast<const bf16x8*>(tile + roff[ks] + h * kHalf);
  }
};

// Copy geometry of one 64-row tile of a [rows][D] tensor: the wavefronts of
// the workgroup split its D/8 copies of 1 KB (4 lines); lane l fills physical
// chunk l % 16 of its line, i.e. the logical (row, chunk) the swizzle puts there.
template <int D, int NW>
struct TileCopy {
  using T = TileLayout<D>;
  static constexpr int kPerWave = (D / 8 + NW - 1) / NW;
  int row[kPerWave], col[kPerWave], dst[kPerWave];
  bool on[kPerWave];
  __device__ __forceinline__ TileCopy(int wave, int lane) {
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int c = wave + NW * i;
      on[i] = c < D / 8;
      const int line = 4 * c + (lane >> 4);
      int k, ch;
      T::at(on[i] ? line : 0, lane & 15, k, ch);
      row[i] = k;
      col[i] = 8 * ch;
      dst[i] = 4 * c * 256;
    }
  }
  // rows past `nrows` read row nrows-1 (in bounds; masked by the caller)
  __device__ __forceinline__ void issue(const __bf16* src, int r0, int nrows, unsigned char* tile) const {
#pragma unroll
    for (int i = 0; i < kPerWave; ++i)
      if (on[i]) {
        const int r = min(r0 + row[i], nrows - 1);
        global_to_lds16(src + (int64_t)r * D + col[i], tile + dst[i]);
      }
  }
};

// 16 bytes per lane from byte voff of the `bytes`-long buffer at src to LDS
// at lds_base + 16 * lane (buffer_load_dwordx4 ... lds).  The hardware checks
// voff against the buffer's length and reads zeros past its end; src and
// bytes are wave-uniform, so the descriptor is built with scalar
// instructions.
__device__ __forceinline__ void buffer_to_lds16(const void* src, uint32_t bytes, int voff, void* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(src), (short)0, (int)bytes, 0x00020000),
      (lds_void*)lds_base, 16, voff, 0, 0, 0);
}

// TileCopy through buffer descriptors: each tile gets a descriptor that
// starts at its first row and ends at row nrows, so the lane's fixed offset
// inside the tile needs no per-tile vector arithmetic and rows past nrows
// read zeros.
template <int D, int NW>
struct TileCopyBuf {
  using T = TileLayout<D>;
  static constexpr int kPerWave = (D / 8 + NW - 1) / NW;
  int voff[kPerWave], dst[kPerWave];
  bool on[kPerWave];
  __device__ __forceinline__ TileCopyBuf(int wave, int lane) {
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int c = wave + NW * i;
      on[i] = c < D / 8;
      const int line = 4 * c + (lane >> 4);
      int k, ch;
      T::at(on[i] ? line : 0, lane & 15, k, ch);
      voff[i] = (k * D + 8 * ch) * 2;
      dst[i] = 4 * c * 256;
    }
  }
  // A tile that starts at or past nrows gets an empty descriptor: the copy
  // reads no memory and fills the tile with zeros.
  __device__ __forceinline__ void issue(const __bf16* src, int nrows, int r0, unsigned char* tile) const {
    const int rb = min(r0, nrows);
    const uint32_t bytes = (uint32_t)(nrows - rb) * (uint32_t)(D * 2);
#pragma unroll
    for (int i = 0; i < kPerWave; ++i)
      if (on[i]) buffer_to_lds16(src + (int64_t)rb * D, bytes, voff[i], tile + dst[i]);
  }
};

// ---------------------------------------------------------------------------
// Launch-order remap for 8 XCDs.
// Consecutive workgroup ids are handed to the XCDs round-robin, and each XCD
// has its own L2.  Mapping hardware id -> logical id so that every XCD gets a
// contiguous range of logical ids keeps the workgroups that share one head's
// K/V on the same L2.  It is a bijection on [0, total) for any total.
// ---------------------------------------------------------------------------
constexpr int kNumXcd = 8;

__device__ __forceinline__ int xcd_remap(int hw_id, int total) {
  const int xcd = hw_id % kNumXcd;
  const int slot = hw_id / kNumXcd;
  const int q = total / kNumXcd;
  const int r = total % kNumXcd;
  return (xcd < r) ? xcd * (q + 1) + slot : r * (q + 1) + (xcd - r) * q + slot;
}

constexpr int kCusPerXcd = 32;

// Work order of the two-workgroups-per-CU kernels.  Each XCD takes a
// contiguous range of R work ids (whole heads when R is a multiple of the
// query tiles per head).  Causal query tiles differ in length, and when the
// grid fits the chip at once (R = two per CU of the XCD), the workgroups in
// positions k and k + R/2 of an XCD share a CU: the first half runs the
// longest tiles of the XCD's heads in decreasing length and the second half
// the rest in increasing length, so every CU gets one long and one short
// tile.  Otherwise the longest tiles go first and the dispatcher balances.
template <bool CAUSAL>
__device__ __forceinline__ void causal_order(int hw_id, int total, int n_qtiles, int& bh, int& qtile) {
  const int lid = xcd_remap(hw_id, total);
  bh = lid / n_qtiles;
  qtile = lid % n_qtiles;
  if (!CAUSAL) return;
  const int xcd = hw_id % kNumXcd, k = hw_id / kNumXcd;
  const int q = total / kNumXcd, r = total % kNumXcd;
  const int R = xcd < r ? q + 1 : q;
  const int start = lid - k;
  if (R == 2 * kCusPerXcd && R % n_qtiles == 0) {
    const int nh = R / n_qtiles;
    const int i = k < R / 2 ? k : R - 1 - (k - R / 2);  // rank in longest-first order
    qtile = n_qtiles - 1 - i / nh;
    bh = start / n_qtiles + i % nh;
  } else {
    qtile = n_qtiles - 1 - qtile;  // longest rows first
  }
}


}  // namespace attn
