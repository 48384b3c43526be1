// FlashDecoding split-K decode for gfx950: one query row per (b, h) against a
// long K/V cache (cnblogs article on FlashAttention tiling, section 3
// scenario B; "FlashAttention 1 和 FlashAttention 2 的区别", sections 6 and 13).
//
// Map step (decode_partial_kernel): one workgroup per (b*h, chunk).  A chunk
// is streamed once from HBM with 16-byte loads issued R keys at a time per
// lane (all loads of a round in flight together); each group of D/8 lanes
// owns one key at a time, forms q.k with bf16 dot2 instructions and a
// cross-lane sum, and keeps a running (m, l, U) over its keys.  The states of
// the key groups are merged across lanes and then across the 4 wavefronts
// with the partial-state merge, and the chunk's (U, m, l) is written to the
// workspace.  This is HBM-bandwidth work: no MFMA (a single query row).
//
// Paged variant: the same kernels, with each key's row found through a block
// table (see PagedKV); the block ids of a round are fetched one round ahead.
//
// Reduce step (decode_merge_kernel): one workgroup per (b, h) merges its S
// partials: m = max m_c, l = sum e^(m_c - m) l_c, U = sum e^(m_c - m) U_c,
// O = U / l, LSE = m + ln l.
#include <atomic>

#include "common.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kRound = 8;  // keys per lane group per round (loads in flight)

struct State {
  float m;  // running max, log2 units of the scaled score
  float l;
  float u[8];
};

// Merge state `o` into `s` (both in log2 units); -inf states carry weight 0.
__device__ __forceinline__ void merge_into(State& s, const State& o) {
  const float mn = fmaxf(s.m, o.m);
  const float ms = (mn == kNegInf) ? 0.f : mn;
  const float a = fast_exp2(s.m - ms);
  const float b = fast_exp2(o.m - ms);
  s.l = a * s.l + b * o.l;
#pragma unroll
  for (int e = 0; e < 8; ++e) s.u[e] = a * s.u[e] + b * o.u[e];
  s.m = mn;
}

__device__ __forceinline__ State shfl_state(const State& s, int mask) {
  State o;
  o.m = shfl_xor_f32(s.m, mask);
  o.l = shfl_xor_f32(s.l, mask);
#pragma unroll
  for (int e = 0; e < 8; ++e) o.u[e] = shfl_xor_f32(s.u[e], mask);
  return o;
}

__device__ __forceinline__ float dot8_bf16(const u32x4& a, const u32x4& b) {
  float acc = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t aw = a[w], bw = b[w];
    acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(aw), as_bf16x2(bw), acc, false);
  }
  return acc;
}

// Where the keys of one (b, h) live.  Dense: row t of the [L, D] slab of
// (b, h).  Paged: row t & (bs - 1) of pool block table[b][t >> log2 bs] of
// head h, the pool laid out [num_blocks][H][bs][D] (the paged block table
// that "FlashAttention 1 和 FlashAttention 2 的区别", section 13, names as a
// KV-cache layout of decode kernels).
struct PagedKV {
  const int32_t* table;    // [B][max_blocks]
  const int32_t* seq_lens; // [B]
  int H, max_blocks, num_blocks, log2_bs;
};

template <int D, bool PAGED>
__global__ __launch_bounds__(kThreads) void decode_partial_kernel(const __bf16* __restrict__ Q,
                                                                  const __bf16* __restrict__ K,
                                                                  const __bf16* __restrict__ V,
                                                                  float* __restrict__ ws, int L, int S,
                                                                  int BH, float scale_log2, PagedKV pg) {
  constexpr int LPK = D / 8;       // lanes per key (8 bf16 each)
  constexpr int SPW = 64 / LPK;    // key slots per wavefront
  constexpr int NS = SPW * kWaves; // key slots per workgroup
  constexpr int STEP = NS * kRound;
  __shared__ float sm_u[kWaves][D];
  __shared__ float sm_ml[kWaves][2];

  // Work order.  Each XCD takes a contiguous range of the work (xcd_remap).
  // Dense: the chunks of one (b, h) are consecutive, so the workgroups in
  // flight stream a few contiguous [L, D] slabs.  Paged: the heads of one
  // chunk are consecutive instead; the pool is block-major, so the H heads of
  // a block are adjacent and an in-order table is read as contiguous runs
  // (head-major order would stride the pool by H blocks and load a few
  // memory channels far more than the rest).
  const int id = xcd_remap(blockIdx.x, BH * S);
  const int bh = PAGED ? id % BH : id / S;
  const int c = PAGED ? id / BH : id % S;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int u = lane % LPK;                    // d chunk: dims 8u .. 8u+7
  const int slot = wave * SPW + lane / LPK;    // key slot in the workgroup

  // Paged: the sequence length comes from seq_lens, clamped to what the
  // table can address, so a bad length or block id never reads outside the
  // pool (the result is then unspecified, not a fault).
  const int32_t* tab = nullptr;
  int h = 0;
  if constexpr (PAGED) {
    const int b = bh / pg.H;
    h = bh - b * pg.H;
    tab = pg.table + (int64_t)b * pg.max_blocks;
    L = min(max(pg.seq_lens[b], 0), pg.max_blocks << pg.log2_bs);
  }
  const int lo = (int)(((int64_t)c * L) / S);
  const int hi = (int)(((int64_t)(c + 1) * L) / S);
  const int bs_mask = (1 << pg.log2_bs) - 1;

  // pool block of each of this lane's keys in the round at k0
  auto fetch_blocks = [&](int k0, int (&blk)[kRound]) {
#pragma unroll
    for (int r = 0; r < kRound; ++r) {
      const int key = k0 + r * NS + slot;
      blk[r] = key < hi ? min(max(tab[key >> pg.log2_bs], 0), pg.num_blocks - 1) : 0;
    }
  };
  // element offset of dims 8u.. of key `key` (in block blk when paged)
  auto row_off = [&](int key, int blk) -> int64_t {
    if constexpr (PAGED)
      return ((((int64_t)blk * pg.H + h) << pg.log2_bs) + (key & bs_mask)) * D + 8 * u;
    else
      return ((int64_t)bh * L + key) * D + 8 * u;
  };

  const u32x4 qv = *reinterpret_cast<const u32x4*>(Q + (int64_t)bh * D + 8 * u);

  State st;
  st.m = kNegInf;
  st.l = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) st.u[e] = 0.f;

  int blk[kRound] = {};
  if constexpr (PAGED) fetch_blocks(lo, blk);
  for (int k0 = lo; k0 < hi; k0 += STEP) {
    u32x4 kr[kRound], vr[kRound];
#pragma unroll
    for (int r = 0; r < kRound; ++r) {
      const int key = k0 + r * NS + slot;
      const bool ok = key < hi;
      const int64_t off = row_off(key, blk[r]);
      // the cache is streamed once: non-temporal loads keep it out of the caches
      kr[r] = ok ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(K + off)) : u32x4{};
      vr[r] = ok ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(V + off)) : u32x4{};
    }
    // block ids of the next round, issued after this round's loads so their
    // latency hides behind this round's arithmetic
    if constexpr (PAGED) fetch_blocks(k0 + STEP, blk);
    float s[kRound];
    float rmax = kNegInf;
#pragma unroll
    for (int r = 0; r < kRound; ++r) {
      float x = dot8_bf16(qv, kr[r]);
#pragma unroll
      for (int msk = 1; msk < LPK; msk <<= 1) x += shfl_xor_f32(x, msk);
      const int key = k0 + r * NS + slot;
      s[r] = key < hi ? x * scale_log2 : kNegInf;
      rmax = fmaxf(rmax, s[r]);
    }
    const float mn = fmaxf(st.m, rmax);
    const float ms = (mn == kNegInf) ? 0.f : mn;
    const float alpha = fast_exp2(st.m - ms);
    st.l *= alpha;
#pragma unroll
    for (int e = 0; e < 8; ++e) st.u[e] *= alpha;
#pragma unroll
    for (int r = 0; r < kRound; ++r) {
      const float p = fast_exp2(s[r] - ms);
      st.l += p;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        st.u[2 * w] = fmaf(p, bf16lo_to_f32(vr[r][w]), st.u[2 * w]);
        st.u[2 * w + 1] = fmaf(p, bf16hi_to_f32(vr[r][w]), st.u[2 * w + 1]);
      }
    }
    st.m = mn;
  }

  // merge the key slots of this wavefront (lanes with equal u)
#pragma unroll
  for (int msk = LPK; msk < 64; msk <<= 1) {
    const State o = shfl_state(st, msk);
    merge_into(st, o);
  }
  if (lane < LPK) {
#pragma unroll
    for (int e = 0; e < 8; ++e) sm_u[wave][8 * u + e] = st.u[e];
    if (lane == 0) {
      sm_ml[wave][0] = st.m;
      sm_ml[wave][1] = st.l;
    }
  }
  __syncthreads();

  // merge the 4 wavefronts and write U [bh][c][d], m [bh][c], l [bh][c]
  if (tid < D) {
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm_ml[w][0]);
    const float Ms = (M == kNegInf) ? 0.f : M;
    float acc = 0.f, lt = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float wt = fast_exp2(sm_ml[w][0] - Ms);
      acc += wt * sm_u[w][tid];
      lt += wt * sm_ml[w][1];
    }
    const int64_t pc = (int64_t)bh * S + c;
    ws[pc * D + tid] = acc;
    if (tid == 0) {
      float* wm = ws + (int64_t)BH * S * D;
      float* wl = wm + (int64_t)BH * S;
      wm[pc] = (M == kNegInf) ? kNegInf : M * kLn2;
      wl[pc] = lt;
    }
  }
}

// Reduce step: one workgroup per (b, h).  Each lane owns 4 consecutive dims
// and a subset of the chunks; it forms the weights e^(m_c - m) of its chunks
// and reads their U_c rows with 16-byte loads, several chunks in flight, and
// the per-dim partial sums are combined through LDS.
template <int D>
__global__ __launch_bounds__(kThreads) void decode_merge_kernel(const float* __restrict__ ws, __bf16* __restrict__ O,
                                                                float* __restrict__ LSE, int S, int BH) {
  constexpr int LPR = D / 4;           // lanes per U row (4 dims each)
  constexpr int RPW = kThreads / LPR;  // chunk rows read together by the workgroup
  constexpr int UNR = 4;               // rows in flight per lane
  __shared__ float sm_red[kThreads];
  __shared__ f32x4 sm_acc[RPW][LPR];

  const int bh = blockIdx.x;
  const int tid = threadIdx.x;
  const float* wu = ws + (int64_t)bh * S * D;
  const float* wm = ws + (int64_t)BH * S * D + (int64_t)bh * S;
  const float* wl = ws + (int64_t)BH * S * D + (int64_t)BH * S + (int64_t)bh * S;

  // M = max_c m_c (natural-log units)
  float mx = kNegInf;
  for (int c = tid; c < S; c += kThreads) mx = fmaxf(mx, wm[c]);
  sm_red[tid] = mx;
  __syncthreads();
  for (int st = kThreads / 2; st > 0; st >>= 1) {
    if (tid < st) sm_red[tid] = fmaxf(sm_red[tid], sm_red[tid + st]);
    __syncthreads();
  }
  const float M = sm_red[0];
  const float Ms = (M == kNegInf) ? 0.f : M;
  __syncthreads();

  auto weight = [&](int c) {
    const float mc = wm[c];
    return (mc == kNegInf) ? 0.f : fast_exp2((mc - Ms) * kLog2e);
  };
  // l = sum_c w_c l_c
  float lpart = 0.f;
  for (int c = tid; c < S; c += kThreads) lpart += weight(c) * wl[c];
  sm_red[tid] = lpart;
  __syncthreads();
  for (int st = kThreads / 2; st > 0; st >>= 1) {
    if (tid < st) sm_red[tid] += sm_red[tid + st];
    __syncthreads();
  }
  const float lt = sm_red[0];

  // U = sum_c w_c U_c
  const int q = tid % LPR, r0 = tid / LPR;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int c0 = r0; c0 < S; c0 += RPW * UNR) {
    f32x4 v[UNR];
    float w[UNR];
#pragma unroll
    for (int k = 0; k < UNR; ++k) {
      const int c = c0 + k * RPW;
      v[k] = c < S ? *reinterpret_cast<const f32x4*>(wu + (int64_t)c * D + 4 * q) : f32x4{};
      w[k] = c < S ? weight(c) : 0.f;
    }
#pragma unroll
    for (int k = 0; k < UNR; ++k) acc += w[k] * v[k];
  }
  sm_acc[r0][q] = acc;
  __syncthreads();
  if (tid < LPR) {
    f32x4 u = sm_acc[0][tid];
#pragma unroll
    for (int r = 1; r < RPW; ++r) u += sm_acc[r][tid];
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    u32x2 o = {pack_bf16x2(u[0] * inv, u[1] * inv), pack_bf16x2(u[2] * inv, u[3] * inv)};
    *reinterpret_cast<u32x2*>(O + (int64_t)bh * D + 4 * tid) = o;
    if (tid == 0 && LSE != nullptr) LSE[bh] = lt > 0.f ? M + fast_log2(lt) * kLn2 : kNegInf;
  }
}

template <int D, bool PAGED>
hipError_t run_decode(const DecodeArgs& a, const PagedKV& pg, hipStream_t s) {
  const int BH = a.B * a.H;
  const int64_t nwg = (int64_t)BH * a.splits;
  hipLaunchKernelGGL((decode_partial_kernel<D, PAGED>), dim3((unsigned)nwg), dim3(kThreads), 0, s,
                     static_cast<const __bf16*>(a.q), static_cast<const __bf16*>(a.k),
                     static_cast<const __bf16*>(a.v), a.ws, a.L, a.splits, BH, a.scale * kLog2e, pg);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_merge_kernel<D>), dim3(BH), dim3(kThreads), 0, s, a.ws, static_cast<__bf16*>(a.o),
                     a.lse, a.splits, BH);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t s) {
  const PagedKV none{nullptr, nullptr, a.H, 0, 0, 0};
  return a.d == 64 ? run_decode<64, false>(a, none, s) : run_decode<128, false>(a, none, s);
}

hipError_t launch_decode_paged_bf16(const DecodeArgs& a, const PagedArgs& p, hipStream_t s) {
  const PagedKV pg{p.block_table, p.seq_lens, a.H, p.max_blocks, p.num_blocks, p.log2_bs};
  return a.d == 64 ? run_decode<64, true>(a, pg, s) : run_decode<128, true>(a, pg, s);
}

// ---------------------------------------------------------------------------
// The decode without allocation.  Its partials go to `scratch`, a fixed array
// that each device holds for the life of the process, so the call needs no
// workspace from the caller.  In host code `scratch` names a host-side
// stand-in, not device memory: its device address is looked up once per
// device with hipGetSymbolAddress and only that address reaches the kernels.
// The partial kernel writes every (U, m, l) entry that the merge kernel reads,
// so nothing has to be cleared between calls.
// ---------------------------------------------------------------------------
namespace {
static __device__ __align__(256) float scratch[kDecodeScratchBytes / sizeof(float)];

constexpr int kMaxDevices = 64;
std::atomic<float*> g_scratch[kMaxDevices];

// Device address of the current device's scratch (looked up on first use).
hipError_t scratch_address(float** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  float* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    void* addr = nullptr;
    e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (addr == nullptr) return hipErrorInvalidSymbol;
    p = static_cast<float*>(addr);
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return hipSuccess;
}
}  // namespace

hipError_t launch_decode_noalloc_bf16(const DecodeArgs& a, hipStream_t s) {
  DecodeArgs b = a;
  hipError_t e = scratch_address(&b.ws);
  if (e != hipSuccess) return e;
  return launch_decode_bf16(b, s);
}

}  // namespace attn
