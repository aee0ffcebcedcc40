// bf16 blockwise step attention on gfx950 matrix cores (one ring step of one
// rank).
//
// What one launch computes ("Sequence Parallelism IV: Megatron Context
// Parallel and Load-Balanced Rings", section 4 "What Actually Moves"): the
// rank's resident queries against the K/V chunks held in one receive slot,
// with the online-softmax state (running max m, running sum l, unnormalised
// O) carried across K/V tiles, so the step's partial (O_s, lse_s) is exact;
// the epilogue folds it into the rank's running state by LSE correction.
// Each query row sees a prefix of the slot (its segment's kv_full keys, plus
// the keys up to its own position on a diagonal chunk); K/V tiles past a
// wave's longest prefix are skipped, which is the skipping of causally
// future sub-blocks of the same section.
//
// gfx950 mapping:
//   * workgroup = 8 waves = 256 query rows of one head for head_dim 128
//     (4 waves = 128 rows for head_dim 64); wave w owns 32 rows.
//   * scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16: A = K from LDS (row = key), B = Q^T from
//     registers (column = query).  The 32x32 result leaves every lane with 16
//     keys of ONE query, so the row max and row sum are per-lane reductions
//     plus a single exchange with the lane 32 away.
//   * O^T = V^T P^T with the same instruction: B = P^T straight from the score
//     registers (converted to bf16, round-to-nearest-even), A = V^T from LDS,
//     with the keys of every 16-key group in the order in which the score
//     registers hold them, so P never leaves registers.
//   * K/V tiles of 64 keys come in with buffer loads (hardware range check:
//     keys past the slot read as zero).  head_dim 64: into registers two
//     tiles ahead, then into a double-buffered LDS tile (K row-major, V
//     transposed; 16-byte padded rows keep the operand reads bank-conflict
//     free).  head_dim 128: straight into a four-stage LDS ring, V row-major
//     and read transposed (see the head_dim 128 kernel below).
//   * softmax in base 2: p = exp2(s * scale * log2 e - m); the reference max m
//     may lag the true max by up to 8 (p <= 2^8), which skips most O rescales
//     and is exact for any choice of m.  The head_dim 128 kernel does not even
//     take a tile's max unless a lane's tile sum exceeds 2^8.
//   * workgroup ids are remapped so consecutive logical tiles (same head, same
//     K/V) share an XCD and its L2; the logical order puts the longest rows of
//     a diagonal segment first.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "epilogue.h"
#include "lds_dma.h"
#include "kernels.h"

namespace cpattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBM = 128;
constexpr int kBN = 64;
constexpr int kThreads = 256;
constexpr float kRescaleSlack = 8.0f;  // log2 units the reference max may lag behind

// Workgroups are handed to the 8 XCDs round-robin; give XCD x a contiguous
// range of logical ids so tiles that share K/V also share an L2.
__device__ __forceinline__ int xcd_remap(int b, int n) {
  const int x = b & 7, slot = b >> 3;
  const int q = n >> 3, r = n & 7;
  return x * q + min(x, r) + slot;
}

// (head, tile) of workgroup b.  When the heads split evenly over the 8 XCDs,
// each XCD owns heads/8 whole heads and walks their tiles tile-major (all its
// heads' first tile, then their second, ...), so the longest tiles of every
// head start first; otherwise heads are walked one after the other.
__device__ __forceinline__ void tile_of(int b, int n, int heads, int tiles, int& h, int& t) {
  if ((heads & 7) == 0) {
    const int hg = heads >> 3;
    const int x = b & 7, slot = b >> 3;
    h = x * hg + slot % hg;
    t = slot / hg;
  } else {
    const int L = xcd_remap(b, n);
    h = L / tiles;
    t = L % tiles;
  }
}

// Column of key offset k (multiple of 4) inside the V^T tile: within each
// 16-key group, offsets 8a + 4b + e live at column 8b + 4a + e.
__device__ __forceinline__ int vt_col(int k) { return (k & ~15) | ((k & 4) << 1) | ((k & 8) >> 1); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  // raw buffer (stride 0): loads at byte offsets >= bytes return zero
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), static_cast<short>(0), static_cast<int>(bytes),
                                           0x00020000);
}

__device__ __forceinline__ unsigned pack_lo(unsigned a, unsigned b) { return (a & 0xffffu) | (b << 16); }
__device__ __forceinline__ unsigned pack_hi(unsigned a, unsigned b) { return (a >> 16) | (b & 0xffff0000u); }

template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(2, 2)))
void attn_step_bf16(StepArgs a) {
  constexpr int KS = D + 8;      // LDS K row stride (bf16)
  constexpr int VS = kBN + 8;    // LDS V^T row stride (bf16)
  constexpr int CPR = D / 8;     // 16-byte chunks per K/V row
  constexpr int KCH = kBN * CPR / kThreads;      // K chunks per thread
  constexpr int VITEMS = (kBN / 4) * CPR;        // (4 keys x 8 dims) items per V tile
  constexpr int NT = D / 16;     // k-steps of the score contraction
  constexpr int NB = D / 32;     // 32-row blocks of O^T
  static_assert(KCH >= 1 && kBN * CPR % kThreads == 0, "K staging");
  static_assert(VITEMS <= kThreads, "V staging");

  __shared__ __attribute__((aligned(16))) uint16_t sk[2][kBN * KS];
  __shared__ __attribute__((aligned(16))) uint16_t sv[2][D * VS];

  int h, t;
  tile_of(blockIdx.x, gridDim.x, a.heads, a.total_tiles, h, t);
  const int si = t < a.seg[0].tiles ? 0 : 1;
  if (si) t -= a.seg[0].tiles;
  const SegArgs& g = a.seg[si];
  const int epi = __builtin_amdgcn_readfirstlane(g.epi);  // scalar: the epilogue branches on it
  if (g.diag) t = g.tiles - 1 - t;  // longest rows first
  const int row0 = t * kBM;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int qc = lane & 31, hf = lane >> 5;
  const int row = row0 + wv * 32 + qc;  // row within the segment
  const bool ok = row < g.q_len;

  const int tile_last = min(row0 + kBM, g.q_len);
  int kv_end = g.kv_full + (g.diag ? tile_last : 0);
  const int w_first = row0 + wv * 32;
  const int w_last = min(w_first + 32, g.q_len);
  const bool w_active = w_last > w_first;
  int w_max = w_active ? g.kv_full + (g.diag ? w_last : 0) : 0;      // longest prefix in the wave
  int w_min = g.kv_full + (g.diag ? w_first + 1 : 0);                // shortest prefix in the wave
  int prefix = ok ? g.kv_full + (g.diag ? row + 1 : 0) : w_max;

  const int64_t hd = int64_t(a.heads) * D;
  const int64_t grow = g.q_global + row;
  // document masks (as in the head_dim 128 kernel below): this row's first
  // key, the wave's smallest and largest first key, the workgroup's first key
  const bool doc = a.doc != nullptr;
  int klo = 0, w_lo = 0, w_lo_last = 0, wg_lo = 0;
  if (doc) {
    int lo, hi;
    doc_row_keys(a, g.q_global + min(row, g.q_len - 1), lo, hi);
    klo = lo;
    prefix = min(prefix, hi);
    doc_row_keys(a, g.q_global + row0, wg_lo, hi);
    doc_row_keys(a, g.q_global + tile_last - 1, lo, hi);
    kv_end = min(kv_end, hi);
    if (w_active) {
      doc_row_keys(a, g.q_global + w_first, w_lo, hi);
      w_min = min(w_min, hi);
      doc_row_keys(a, g.q_global + w_last - 1, w_lo_last, hi);
      w_max = min(w_max, hi);
    }
  }

  // Q^T operand: lane holds Q[row][16 t + 8 hf + 0..7].
  bf16x8 qf[NT];
  {
    const __bf16* qp = static_cast<const __bf16*>(a.q) + grow * hd + int64_t(h) * D + 8 * hf;
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      if (ok) {
        qf[i] = *reinterpret_cast<const bf16x8*>(qp + 16 * i);
      } else {
        qf[i] = bf16x8{};
      }
    }
  }

  f32x16 o[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) o[b] = f32x16{};
  float m = -INFINITY, l = 0.f;

  // K/V reads go through buffer resources with 32-bit offsets.
  const uint32_t row_bytes = uint32_t(a.heads) * D * 2;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.k, uint32_t(a.kv_bytes));
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(a.v, uint32_t(a.kv_bytes));
  const uint32_t head_off = uint32_t(h) * D * 2;

  u32x4 kreg[KCH];
  u32x4 vreg[4];
  // V item of this thread: keys 4 vkg .. 4 vkg + 3, dims 8 vdg .. 8 vdg + 7.
  // Sixteen consecutive lanes take sixteen key groups of one dim group, so
  // their 8-byte transposed writes land on sixteen different bank pairs.
  const int vkg = tid & 15, vdg = tid >> 4;

  // keys past the source's real keys are clamped to its last real row (and masked)
  auto src_off = [&](int kk) { return uint32_t(kv_row(a, min(kk, a.kv_valid - 1))) * row_bytes + head_off; };
  auto load_tile = [&](int j0) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = tid + kThreads * i;
      const int kr = c / CPR, cc = c % CPR;
      kreg[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, src_off(j0 + kr) + cc * 16, 0, 0);
    }
    if (tid < VITEMS) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        vreg[e] = __builtin_amdgcn_raw_buffer_load_b128(rv, src_off(j0 + 4 * vkg + e) + vdg * 16, 0, 0);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = tid + kThreads * i;
      const int kr = c / CPR, cc = c % CPR;
      *reinterpret_cast<u32x4*>(&sk[buf][kr * KS + cc * 8]) = kreg[i];
    }
    if (tid < VITEMS) {
      const int col = vt_col(4 * vkg);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        u32x2 lo, hi;
        lo[0] = pack_lo(vreg[0][w], vreg[1][w]);
        lo[1] = pack_lo(vreg[2][w], vreg[3][w]);
        hi[0] = pack_hi(vreg[0][w], vreg[1][w]);
        hi[1] = pack_hi(vreg[2][w], vreg[3][w]);
        *reinterpret_cast<u32x2*>(&sv[buf][(8 * vdg + 2 * w) * VS + col]) = lo;
        *reinterpret_cast<u32x2*>(&sv[buf][(8 * vdg + 2 * w + 1) * VS + col]) = hi;
      }
    }
  };

  // Double-buffered LDS: tile it is read from buffer it&1 while tile it+1 is
  // written to the other buffer and tile it+2 is in flight in registers; one
  // barrier per tile.
  const int kb0 = (doc ? wg_lo / kBN : 0) * kBN;  // first key tile of the workgroup
  const int ntiles = max(0, (kv_end + kBN - 1) / kBN - kb0 / kBN);
  if (ntiles > 0) {
    load_tile(kb0);
    store_tile(0);
  }
  if (ntiles > 1) load_tile(kb0 + kBN);
  __syncthreads();
  int done = 0;  // key tiles this wave scored (work counter)
  for (int it = 0; it < ntiles; ++it) {
    const int j0 = kb0 + it * kBN;
    const int buf = it & 1;
    if (j0 < w_max && (!doc || j0 + kBN > w_lo)) {
      ++done;
      const uint16_t* skb = sk[buf];
      const uint16_t* svb = sv[buf];
      // S^T tile: s[kb][i] = score(key j0 + 32 kb + 8 (i/4) + 4 hf + i%4, query row)
      f32x16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = f32x16{};
#pragma unroll
        for (int i = 0; i < NT; ++i) {
          const bf16x8 ka = *reinterpret_cast<const bf16x8*>(&skb[(32 * kb + qc) * KS + 16 * i + 8 * hf]);
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[i], s[kb], 0, 0, 0);
        }
      }
      if (j0 + kBN > w_min || (doc && j0 < w_lo_last)) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = j0 + 32 * kb + 8 * (i >> 2) + 4 * hf + (i & 3);
            if (key >= prefix || (doc && key < klo)) s[kb][i] = -INFINITY;
          }
        }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mt = mx * a.scale_log2;
      if (__any(mt > m + kRescaleSlack)) {
        const float mn = fmaxf(m, mt);
        const float alpha = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m - mn);
        l *= alpha;
#pragma unroll
        for (int b = 0; b < NB; ++b) o[b] *= alpha;
        m = mn;
      }
      const float mref = (m == -INFINITY) ? 0.f : m;
      bf16x8 pb[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][i], a.scale_log2, -mref));
          l += p;
          pb[kb][i >> 3][i & 7] = static_cast<__bf16>(p);
        }
      }
      // O^T += V^T P^T over the 64 keys, 16 at a time
#pragma unroll
      for (int b = 0; b < NB; ++b) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const bf16x8 va =
                *reinterpret_cast<const bf16x8*>(&svb[(32 * b + qc) * VS + 32 * kb + 16 * u + 8 * hf]);
            o[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[kb][u], o[b], 0, 0, 0);
          }
        }
      }
    }
    if (it + 1 < ntiles) {
      store_tile(buf ^ 1);
      if (it + 2 < ntiles) load_tile(kb0 + (it + 2) * kBN);
    }
    __syncthreads();
  }

  if (a.tile_cnt && lane == 0)
    __hip_atomic_fetch_add(a.tile_cnt, (unsigned long long)done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  l += __shfl_xor(l, 32);
  if (!ok) return;
  const int lrow = g.q_start + row;
  const float lse_s = (m + __builtin_amdgcn_logf(l)) * 0.69314718055994530942f;
  const float inv = l > 0.f ? 1.f / l : 0.f;  // a row that saw no key (document masks): O_s = 0, lse_s = -inf
  if (doc && l == 0.f && epi == kEpiMerge) return;  // ... and leaves a merge-only step's running state as it is
  float4 c[NB][4];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) c[b][q4] = row_epi_load4(a, epi, h, lrow, 32 * b + 8 * q4 + 4 * hf, D);
  const RowEpi e = row_epi_begin(a, epi, h, lrow, lse_s);
#pragma unroll
  for (int b = 0; b < NB; ++b) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const float4 v4 = make_float4(o[b][4 * q4] * inv, o[b][4 * q4 + 1] * inv, o[b][4 * q4 + 2] * inv,
                                    o[b][4 * q4 + 3] * inv);
      row_epi_store4(a, epi, e, h, lrow, grow, 32 * b + 8 * q4 + 4 * hf, D, v4, c[b][q4]);
    }
  }
  if (hf == 0) row_epi_store_lse(a, epi, e, h, lrow, grow, lse_s);
}

// ---------------------------------------------------------------------------
// head_dim 128: direct-to-LDS K/V, four LDS stages, eight waves.
//
//   * K/V tiles of 64 keys move global -> LDS with buffer_load ... lds (no
//     register staging); each wave instruction fills four 256-byte rows, and
//     the 16-byte chunks of a row are XOR-swizzled (swz) so that both the
//     K operand reads (32 rows, one chunk) and the transposed V reads below
//     hit distinct LDS banks.
//   * V stays row-major in LDS and is read with ds_read_b64_tr_b16: within a
//     16-lane group, lane i receives element i%4 of the 8 bytes addressed by
//     lane 4j + i/4 as its j-th value, so the 16 lanes that point at 4 key
//     rows x 4 column pieces receive 4 keys of one head-dim column each --
//     exactly the A operand of O^T = V^T P^T.
//   * Matrix operands are read from LDS in batches ahead of their MFMAs (all
//     16 K fragments of a tile; V in groups of four), pinned with
//     scheduling-group barriers.
// ---------------------------------------------------------------------------

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;

constexpr int kTileBytes = kBN * 256;  // one 64-key K or V tile of 128 bf16 columns

// Permutation of the 16 chunks of a 256-byte row (linear over GF(2) in the
// row index): bit0 <- r2, bit1 <- r1^r3, bit2 <- r0, bit3 <- r1.
__device__ __forceinline__ int swz(int r) {
  return ((r >> 2) & 1) | ((((r >> 1) ^ (r >> 3)) & 1) << 1) | ((r & 1) << 2) | (((r >> 1) & 1) << 3);
}

__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

// Workgroup barrier ordering LDS only.  __syncthreads() also orders global
// memory, which makes every wave wait for all of its global loads and stores
// in flight (the ring copy included); LDS written by direct-to-LDS loads is
// covered by each wave's own vmcnt wait before the barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS accesses are done
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);  // no compiler reordering of memory accesses across
}

// ---------------------------------------------------------------------------
// Eight waves: 256 query rows per workgroup, 32 per wave (one workgroup per
// CU, still two waves per SIMD).  Every K/V tile in LDS serves 256 rows, so
// the loads per flop are half those of a four-wave workgroup; four K/V
// stages: tile j+2 is loaded while tile j computes, two tiles of latency.
//
// Ring receive (kRecv): the workgroup's share of the next step's K/V is cut
// into ntiles chunks of at most 256 16-byte vectors.  The waves of group A
// (0-3) copy one chunk per tile through registers, at the start of tile j:
// chunk j - 1 (loaded at the start of tile j - 1, a whole tile earlier, so
// the wait before its store finds it landed) is stored and chunk j loaded.
// Every A wave issues exactly one copy store and one copy load per tile
// (lanes with nothing to copy repeat a vector of the share: the same bytes
// to the same place), so its end-of-tile wait for tile j + 1 stays a fixed
// count of younger loads, vmcnt(5).  Group B copies nothing.  What does not
// fit in the chunks is copied after the loop.  (An earlier form staged the
// copy through LDS with direct-to-LDS loads in every wave; each such load
// holds its wave at issue for about 50 clocks, and the copy cost more.)
//
// Document masks (kDoc): a row sees only the run of the source's keys that
// holds its own document, [klo, khi), clipped to its prefix.  The rows of a
// segment are consecutive positions, so klo and khi grow with the row: a
// run of rows takes its first key from its first row and its last from its
// last row.  The workgroup starts at the 64-key tile of its first row's klo,
// a wave skips the tiles below its first row's klo, and tiles that reach
// below its last row's klo are masked.
// ---------------------------------------------------------------------------

constexpr int kThreads8 = 512;
constexpr int kBM8 = 256;

// Fused-ring receive wait: poll flag `step` of the call until it reaches the
// call's epoch `ep` (wrap-aware), sleeping between polls; after ring_polls polls
// the wave's first lane records the time-out in the host-visible word and
// the wave goes on.  The relaxed agent-scope load reads the flag through to
// device coherence (sc1), never from an older copy in this XCD's L2.  Every
// lane of the calling wave takes the same path.
__device__ __forceinline__ void ring_wait(const StepArgs& a, int step, uint32_t ep) {
  const uint32_t* const f = a.ring_flags + step;
  for (int n = 0; int32_t(__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) - ep) < 0; ++n) {
    if (n >= a.ring_polls) {
      if ((threadIdx.x & 63) == 0) __hip_atomic_store(a.ring_err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      break;
    }
    __builtin_amdgcn_s_sleep(8);
  }
}

// kRanks: every rank's step of one ring step in one launch (a CP group in
// lockstep on one GPU): rank r's workgroups are wgb[r] .. wgb[r + 1] - 1
// (ranges that start at multiples of 8, so a rank's workgroups keep their
// XCD mapping), its arguments tbl[r] (device memory); a workgroup past its
// rank's tiles (padding of the range) does nothing.  Otherwise the launch is
// one rank's step, with arguments a0.
// kRing: every ring step of one rank in one launch.  A row tile's keys are
// the runs of its segment (StepArgs::runs): the rank's own chunks in place
// and the receive slots of steps 1 .. P-1, every run a whole number of
// 64-key tiles, the causal diagonal last.  The running max and sum stay in
// registers from the first step to the last, and the epilogue writes the
// output once.  At the top of tile j (j a multiple of 4) wave 4 holds the
// workgroup until the receives of the runs up to tile j + 6 have landed
// (their flags carry the call's epoch); the barrier that ends tile j puts
// that ahead of every load of tiles j + 3 .. j + 6, which the waves issue in
// tiles j + 1 .. j + 4.  No cache maintenance
// is needed: a slot's rows reach a cache of this kernel only through those
// loads, after the flag; the kernel started with its caches invalidated
// (kernel-start acquire), and the copy kernel's writes were made visible at
// agent scope when it completed, before the signal kernel behind it on the
// copy stream stored the flag.
template <bool kRecv, bool kDoc, bool kRanks, bool kRing = false>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads8, kThreads8), amdgpu_waves_per_eu(2, 2)))
void attn_step_bf16_d128x8(StepArgs a0, const StepArgs* __restrict__ tbl, const int32_t* __restrict__ wgb, int nranks) {
  constexpr int D = 128, NT = 8, NB = 4;
  static_assert(!(kRanks && kRecv), "the in-kernel receive is per rank");
  static_assert(!(kRing && (kRecv || kDoc || kRanks)), "the fused ring stands alone");
  int bid = int(blockIdx.x), nblk = int(gridDim.x), rank = 0;
  if constexpr (kRanks) {
    int lo = 0, hi = nranks;  // the rank: wgb[lo] <= blockIdx.x < wgb[lo + 1]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (wgb[mid] <= bid) lo = mid;
      else hi = mid;
    }
    rank = lo;
    bid -= wgb[lo];
    nblk = tbl[lo].total_tiles * tbl[lo].heads;
    if (bid >= nblk) return;
  }
  const StepArgs& a = kRanks ? tbl[rank] : a0;
  // 4 stages x K, V
  __shared__ __attribute__((aligned(1024))) uint8_t smem_kv[4 * 2 * kTileBytes];
  lds_u8* const kv_lds = (lds_u8*)smem_kv;
  // the four K stages fill the first 64 KiB, the four V stages the second:
  // with a constant stage every operand read addresses a per-lane base plus
  // an offset below 64 KiB, which the read instruction carries itself
  auto kst = [&](int st) { return kv_lds + st * kTileBytes; };
  auto vst = [&](int st) { return kv_lds + (4 + st) * kTileBytes; };
  // The transposed V reads take no offset from the compiler: a constant V
  // stage would only make it keep every stage's eight addresses in VGPRs.
  // The stage base goes through an SGPR the compiler cannot see into (an
  // empty assembly statement), so each read adds it, as with a loop index.
  auto vst_rt = [&](int st) {
    int o = (4 + st) * kTileBytes;
    asm volatile("" : "+s"(o));
    return kv_lds + o;
  };

  int h, t;
  tile_of(bid, nblk, a.heads, a.total_tiles, h, t);
  const int si = t < a.seg[0].tiles ? 0 : 1;
  if (si) t -= a.seg[0].tiles;
  const SegArgs& g0 = a.seg[si];
  // key split: a full segment on a grid smaller than the GPU is cut into
  // ksplit = 2 key ranges per row tile, one workgroup each (adjacent ids);
  // in the fused ring each part has its own run list, part 1's in seg[si + 2]
  const int ks = g0.ksplit;
  const int part = t % ks;
  t /= ks;
  if (g0.diag || (kRing && ks > 1)) t = g0.tiles / ks - 1 - t;  // longest rows first
  const SegArgs& g = (kRing && part) ? a.seg[si + 2] : g0;
  const int epi = __builtin_amdgcn_readfirstlane(g.epi);  // scalar: the epilogue branches on it
  const int row0 = t * kBM8;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keep wave-level values scalar
  const int qc = lane & 31, hf = lane >> 5;
  const int row = row0 + wv * 32 + qc;
  const bool ok = row < g.q_len;
  const int tile_last = min(row0 + kBM8, g.q_len);
  int kv_end = g.kv_full + (g.diag ? tile_last : 0);
  const int w_first = row0 + wv * 32;
  const int w_last = min(w_first + 32, g.q_len);
  int w_max = w_last > w_first ? g.kv_full + (g.diag ? w_last : 0) : 0;
  int w_min = g.kv_full + (g.diag ? w_first + 1 : 0);
  int prefix = ok ? g.kv_full + (g.diag ? row + 1 : 0) : w_max;
  const int64_t hd = int64_t(a.heads) * D;
  const int64_t grow = g.q_global + row;
  // document masks: this row's first key, the wave's smallest and largest
  // first key, the workgroup's first key
  int klo = 0, w_lo = 0, w_lo_last = 0, wg_lo = 0;
  if constexpr (kDoc) {
    int lo, hi;
    doc_row_keys(a, g.q_global + min(row, g.q_len - 1), lo, hi);
    klo = lo;
    prefix = min(prefix, hi);
    doc_row_keys(a, g.q_global + row0, wg_lo, hi);
    doc_row_keys(a, g.q_global + tile_last - 1, lo, hi);
    kv_end = min(kv_end, hi);
    if (w_last > w_first) {
      doc_row_keys(a, g.q_global + w_first, w_lo, hi);
      w_min = min(w_min, hi);
      doc_row_keys(a, g.q_global + w_last - 1, w_lo_last, hi);
      w_max = min(w_max, hi);
    }
  }
  // whether the wave computes the key tile at j0
  auto live = [&](int j0) { return j0 < w_max && (!kDoc || j0 + kBN > w_lo); };

  bf16x8 qf[NT];
  {
    const __bf16* qp = static_cast<const __bf16*>(a.q) + grow * hd + int64_t(h) * D + 8 * hf;
#pragma unroll
    for (int i = 0; i < NT; ++i) qf[i] = ok ? *reinterpret_cast<const bf16x8*>(qp + 16 * i) : bf16x8{};
  }
  f32x16 o[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) o[b] = f32x16{};
  float m = -INFINITY, l = 0.f;

  // load mapping (waves 0-3 load every tile): wave wv, instruction n fills
  // tile rows 16 wv + 4 n + lane/16; the lane's 16 bytes land in physical
  // chunk lane%16 of that row.  swz is linear over GF(2) and reads the row's
  // low four bits only, and lane/16 and 4 n have disjoint bits, so the chunk
  // of instruction n is (lane%16 ^ swz(lane/16)) ^ swz(4 n).
  const uint32_t row_bytes = uint32_t(a.heads) * 256;
  const int lrow0 = 16 * (wv & 3) + (lane >> 4);
  const uint32_t hbase = uint32_t(h) * 256 + (((lane & 15) ^ swz(lane >> 4)) << 4);
  uint32_t vrow[4];  // per-lane byte offset of its chunk within a tile whose rows are contiguous
#pragma unroll
  for (int n = 0; n < 4; ++n) vrow[n] = uint32_t(lrow0 + 4 * n) * row_bytes + (hbase ^ (uint32_t(swz(4 * n)) << 4));
  const u32x4 desc_k = buffer_desc(a.k, uint32_t(a.kv_bytes));
  const u32x4 desc_v = buffer_desc(a.v, uint32_t(a.kv_bytes));
  // fused ring: the wave's position in the segment's key runs and the buffer
  // of its current run (a wave loads only K or only V: one descriptor); wave
  // 0 keeps a second position for the receive gate
  int ld_run = -1, ld_end = 0, ld_delta = 0;
  u32x4 ld_desc = {};
  // the run table is written once at set-up and only read here: through the
  // constant address space its wave-uniform reads are scalar loads
  typedef const __attribute__((address_space(4))) RingRun c_run;
  c_run* const runs = (c_run*)(a.runs);
  uint32_t gt_epoch = 0;  // (wave 4) the call's epoch, read before the first wait
  int gt_run = -1, gt_end = 0, gt_step = 0;
  auto gate = [&](int j0) {  // wave 4: the receives of the runs up to the one holding key j0 have landed
    while (j0 >= gt_end) {
      ++gt_run;
      c_run& rr = runs[g.run0 + gt_run];
      gt_end = __builtin_amdgcn_readfirstlane(rr.end);  // (wave-uniform: keep run fields scalar)
      const int st = __builtin_amdgcn_readfirstlane(rr.step);
      if (st > gt_step) {
        if (gt_step == 0) {
          // written by the kernel before this launch on its stream: the
          // constant address space reads it with a scalar load
          typedef const __attribute__((address_space(4))) uint32_t c_u32;
          gt_epoch = *(c_u32*)(a.ring_flags) + a.ring_epoch_add;
        }
        ring_wait(a, st, gt_epoch);
        gt_step = st;
      }
    }
  };
  auto issue = [&](const u32x4& desc, int j0, lds_u8* dst) {
    if constexpr (kRing) {
      // runs are whole tiles: the tile's 64 rows are consecutive rows of one buffer
      while (j0 >= ld_end) {
        ++ld_run;
        c_run& rr = runs[g.run0 + ld_run];
        ld_end = __builtin_amdgcn_readfirstlane(rr.end);
        ld_delta = __builtin_amdgcn_readfirstlane(rr.delta);
        if (__builtin_amdgcn_readfirstlane(rr.buf))
          ld_desc = buffer_desc(wv < 4 ? a.k2 : a.v2, uint32_t(a.kv2_bytes));
        else
          ld_desc = buffer_desc(wv < 4 ? a.k : a.v, uint32_t(a.kv_bytes));
      }
      const uint32_t soff = __builtin_amdgcn_readfirstlane(uint32_t(j0 + ld_delta) * row_bytes);
#pragma unroll
      for (int n = 0; n < 4; ++n) dma_lds16(ld_desc, vrow[n], soff, lds_addr(dst + (16 * (wv & 3) + 4 * n) * 256));
      return;
    }
    // Fast path: the 64 source rows are consecutive and inside the buffer, so
    // the tile base is one scalar offset.  Otherwise (a tile that crosses the
    // split between the two chunks, or the ragged last tile) each lane maps
    // its own row and clamps keys past the source's real keys to its last
    // real row (masked).
    const bool whole = j0 + kBN <= a.kv_valid && (j0 + kBN <= a.kv_split || j0 >= a.kv_split);
    if (whole) {
      const uint32_t soff = __builtin_amdgcn_readfirstlane(uint32_t(kv_row(a, j0)) * row_bytes);
#pragma unroll
      for (int n = 0; n < 4; ++n) dma_lds16(desc, vrow[n], soff, lds_addr(dst + (16 * (wv & 3) + 4 * n) * 256));
    } else {
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const int kk = min(j0 + lrow0 + 4 * n, a.kv_valid - 1);
        const uint32_t voff = uint32_t(kv_row(a, kk)) * row_bytes + (hbase ^ (uint32_t(swz(4 * n)) << 4));
        dma_lds16(desc, voff, 0u, lds_addr(dst + (16 * (wv & 3) + 4 * n) * 256));
      }
    }
  };
  // K operand: row 32 kb + qc, logical chunk 2 i + hf.  The chunk bits of
  // 2 i and of hf are disjoint, so the swizzled address is kbase ^ (32 i).
  const uint32_t kbase = qc * 256 + ((hf ^ swz(qc & 15)) << 4);
  // transposed V reads: lane (group g, index i16) points at row 8 r + 4 hf + i16/4 of a 16-key
  // group, bytes 64 b + 32 (g & 1) + 8 (i16 & 3) .. +7; the 64 b part only flips chunk bits 2-3,
  // so the address is vbase[r] ^ (64 b).
  const int i16 = lane & 15, g1 = (lane >> 4) & 1;
  uint32_t vbase[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int vr = 8 * r + 4 * hf + (i16 >> 2);
    const int c0 = 2 * g1 + ((i16 & 3) >> 1);
    vbase[r] = vr * 256 + ((c0 ^ swz(vr & 15)) << 4) + 8 * (i16 & 1);
  }

  // Operand reads are issued in batches ahead of the MFMAs that use them
  // (pinned with scheduling-group barriers), so the matrix cores do not wait
  // for one LDS round trip per instruction.
  auto scores = [&](const lds_u8* kt, f32x16 (&s)[2]) {
    bf16x8 kf[2][NT];
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) kf[kb][i] = *reinterpret_cast<const lds_bf16x8*>(kt + kb * 32 * 256 + (kbase ^ (32u * i)));
    s[0] = f32x16{};
    s[1] = f32x16{};
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kb][i], qf[i], s[kb], 0, 0, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);  // 16 LDS reads first
    __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);  // then 16 MFMAs
  };
  auto softmax = [&](f32x16 (&s)[2], int j0, bf16x8 (&pb)[2][2]) {
    if (j0 + kBN > w_min || (kDoc && j0 < w_lo_last)) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = j0 + 32 * kb + 8 * (i >> 2) + 4 * hf + (i & 3);
          if (key >= prefix || (kDoc && key < klo)) s[kb][i] = -INFINITY;
        }
    }
    float lk[2];  // two partial row sums: half the dependent adds
    auto exps = [&](float mref) {
      lk[0] = lk[1] = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][i], a.scale_log2, -mref));
          lk[kb] += p;
          pb[kb][i >> 3][i & 7] = static_cast<__bf16>(p);
        }
    };
    // Fast path: exponentiate against the running reference max without
    // taking the tile's max.  It stands if no probability exceeds
    // 2^kRescaleSlack, which a lane's tile sum of at most that guarantees
    // (the terms are not negative; an overflow makes the sum infinite).
    // Otherwise, and before any reference exists, the tile's max is taken,
    // the reference moves up to it and the exponentials are redone.
    bool redo = __any(m == -INFINITY);
    if (!redo) {
      exps(m);
      redo = __any(lk[0] + lk[1] > exp2f(kRescaleSlack));
    }
    if (redo) {
      // two independent chains (one per 32-key block), then the lane 32 away
      // through v_permlane32_swap (a VALU exchange, no LDS round trip)
      float mx0 = s[0][0], mx1 = s[1][0];
#pragma unroll
      for (int i = 1; i < 16; ++i) {
        mx0 = fmaxf(mx0, s[0][i]);
        mx1 = fmaxf(mx1, s[1][i]);
      }
      float mx = fmaxf(mx0, mx1);
      {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      }
      const float mn = fmaxf(m, mx * a.scale_log2);
      if (__any(mn > m)) {
        const float alpha = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m - mn);
        l *= alpha;
#pragma unroll
        for (int b = 0; b < NB; ++b) o[b] *= alpha;
        m = mn;
      }
      exps(m == -INFINITY ? 0.f : m);
    }
    l += lk[0] + lk[1];
  };
  auto pv = [&](const lds_u8* vt, const bf16x8 (&pb)[2][2]) {
    // four groups (kb, u) of four head-dim blocks; group g+1's transposed
    // reads are in flight while group g's MFMAs run
    bf16x8 va[4][NB];
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int kb = gq >> 1, u = gq & 1;
      const int roff = (32 * kb + 16 * u) * 256;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vt + roff + (vbase[0] ^ (64u * b))));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vt + roff + (vbase[1] ^ (64u * b))));
        va[gq][b] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    }
#pragma unroll
    for (int gq = 0; gq < 4; ++gq)
#pragma unroll
      for (int b = 0; b < NB; ++b) o[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[gq][b], pb[gq >> 1][gq & 1], o[b], 0, 0, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);  // groups 0 and 1 read
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);   // group 0 MFMAs
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);   // group 2 read
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);   // group 1 MFMAs
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);   // group 3 read
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);   // groups 2 and 3 MFMAs
  };

  // ---- ring receive ----
  // Workgroup b copies from one range, r = b mod n, an even share of that
  // range among the workgroups assigned to it: the source and destination
  // bases are then workgroup-uniform, picked once.  A grid with fewer
  // workgroups than ranges copies whole ranges after the loop instead.
  const int nr = max(a.recv.n, 1);
  const bool whole_ranges = int(gridDim.x) < nr;
  const int rr = int(blockIdx.x) % nr;
  const int64_t rn = rr == 0 ? a.recv.vec[0] : rr == 1 ? a.recv.vec[1] : rr == 2 ? a.recv.vec[2] : a.recv.vec[3];
  const int64_t rg = whole_ranges ? 1 : (int64_t(gridDim.x) - rr + nr - 1) / nr;  // workgroups copying range rr
  const int64_t rsh = (rn + rg - 1) / rg;
  const int64_t rbeg = whole_ranges ? 0 : min(rn, int64_t(blockIdx.x / nr) * rsh);
  const int64_t rend = whole_ranges ? 0 : min(rn, rbeg + rsh);
  typedef __attribute__((address_space(1))) u32x4 g_u32x4;  // global memory: no flat accesses
  const void* const csrc_p = rr == 0 ? a.recv.src[0] : rr == 1 ? a.recv.src[1] : rr == 2 ? a.recv.src[2] : a.recv.src[3];
  g_u32x4* const cdst = (g_u32x4*)(rr == 0 ? a.recv.dst[0] : rr == 1 ? a.recv.dst[1] : rr == 2 ? a.recv.dst[2] : a.recv.dst[3]);
  const g_u32x4* const csrc = (const g_u32x4*)csrc_p;
  // this workgroup's key tiles: jt0 .. jt0 + ntiles - 1 (key kb0 onwards)
  // (document masks: from the tile of the workgroup's first key, never split)
  const int ntiles_all = (kv_end + kBN - 1) / kBN;
  const int half_tiles = (ntiles_all + 1) >> 1;
  // (fused ring: each part has its own run list and key space, from key 0;
  // the zero stays opaque to the compiler, which otherwise keeps more load
  // addresses live and goes past the register budget)
  int jt0 = kDoc ? wg_lo / kBN : (part && !kRing) ? half_tiles : 0;
  if constexpr (kRing) asm volatile("" : "+s"(jt0));
  const int ntiles = kDoc ? max(0, ntiles_all - jt0)
                          : (ks == 1 || kRing) ? ntiles_all : (part ? ntiles_all - half_tiles : half_tiles);
  const int kb0 = jt0 * kBN;
  // chunks of the share: ntiles, at most 256 vectors (one per lane of group
  // A) each; what does not fit is copied after the loop
  const int64_t cv = ntiles > 0 ? min<int64_t>(256, (rend - rbeg + ntiles - 1) / ntiles) : 0;  // vectors per chunk
  // vector of lane a (0..255 over group A) in chunk c: lanes past the chunk
  // repeat its last vector; an empty chunk repeats the share's (or, for an
  // empty share, the range's) last vector
  auto chunk_vec = [&](int64_t c) {
    const int64_t lo = rbeg + c * cv;
    const int64_t hi = min(lo + cv, rend);
    const int64_t fb = rend > rbeg ? rend - 1 : rn - 1;
    return hi > lo ? min(lo + int64_t(wv * 64 + lane), hi - 1) : fb;
  };
  u32x4 creg = {};  // group A: the chunk loaded at the end of the previous tile
  auto copy_step = [&](int j) {
    if (j > 0) __builtin_nontemporal_store(creg, cdst + chunk_vec(j - 1));
    creg = __builtin_nontemporal_load(csrc + chunk_vec(j));
  };

  // Tile j's K/V live in stage j % 4; waves 0-3 load the K tiles and waves
  // 4-7 the V tiles (issue() above), tile j + 2 during tile j.  Every tile
  // load is issued by dma_lds16, so the only waits are these: the prologue
  // waits for all, the end of tile j for all but the loads the wave issued
  // during tile j (four tile loads; with a receive, group A also issued one
  // copy store and one copy load at the start of the tile), so that tile
  // j + 1 has landed.  Loads complete in order among themselves, and a store
  // may complete before older loads: the count 5 of group A with a receive
  // holds back only loads younger than the tile loads of tile j - 1 (the
  // copy load and the four tile loads of tile j; with one of tile j - 1's
  // loads still in flight those five would be too, six or seven in all).
  if constexpr (kRing) {
    // the first three tiles' receives, before the first loads
    if (wv == 4 && ntiles > 0) gate(kb0 + min(2, ntiles - 1) * kBN);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
  }
  if (ntiles > 0) {
    const u32x4& desc = wv < 4 ? desc_k : desc_v;
    issue(desc, kb0, wv < 4 ? kst(0) : vst(0));
    issue(desc, kb0 + min(1, ntiles - 1) * kBN, wv < 4 ? kst(1) : vst(1));
  }
  wait_vmem();
  lds_barrier();

  // Ping-pong: the two waves of a SIMD (wave w and wave w + 4) run half a
  // tile apart, so that one runs its MFMAs while the other runs its softmax.
  // Within tile j:
  //   waves 0-3: product of tile j - 1 and scores of tile j (32 MFMAs), then
  //              softmax of tile j and the loads of K tile j + 2
  //   waves 4-7: softmax of tile j - 1 and the loads of V tile j + 2, then
  //              product of tile j - 1 and scores of tile j
  // with one workgroup barrier per tile, at its end (a second one between
  // the halves only forced the alignment and measured slower).  The loads go
  // to stage (j + 2) % 4: its K tile (j - 2) was last read in tile j - 2 and
  // its V tile in tile j - 1, both before the previous end-of-tile barrier.
  // A direct-to-LDS load holds its wave at issue until the CU's address unit
  // takes it, so the loads come from the softmax half of each wave's tile.
  // Each group runs its own copy of the loop (the barriers pair up by count,
  // not by address), so each copy's registers follow its own live values.
  // Stage and copy-staging indices are loop variables: unrolling to make them
  // constants needs several sets of stage addresses and spills the Q
  // fragments.
  // the MFMA phase of tile J: product of tile J - 1 (probabilities pb_),
  // scores of tile J into s_
#define CPATTN_X8_GEMMS(J, S, s_, pb_)                                                     \
  do {                                                                                     \
    const bool sc_ = live(kb0 + (J) * kBN);                                                \
    const bool pv_ = (J) > 0 && live(kb0 + ((J) - 1) * kBN);                               \
    if (pv_) pv(vst_rt(((S) + 3) & 3), pb_);                                               \
    if (sc_) scores(kst(S), s_);                                                           \
  } while (0)
#define CPATTN_X8_END_A(J)                                                                 \
  do {                                                                                     \
    if constexpr (kRecv)                                                                   \
      __builtin_amdgcn_s_waitcnt(0x0F75); /* vmcnt(5) */                                   \
    else                                                                                   \
      __builtin_amdgcn_s_waitcnt(0x0F74); /* vmcnt(4) */                                   \
    lds_barrier();                                                                         \
  } while (0)
#define CPATTN_X8_END_B()                                                                  \
  do {                                                                                     \
    __builtin_amdgcn_s_waitcnt(0x0F74); /* vmcnt(4) */                                     \
    lds_barrier();                                                                         \
  } while (0)

  // The loops run four tiles per iteration, one per stage, so that each
  // tile's stage is a constant.
  bf16x8 pb_[2][2];  // probabilities of the last softmaxed tile
  f32x16 s_[2];      // scores of the last scored tile
#define CPATTN_X8_TILE_A(J, ST)                                                            \
  do {                                                                                     \
    if ((J) < ntiles) {                                                                    \
      if constexpr (kRecv) copy_step(J);                                                   \
      CPATTN_X8_GEMMS(J, ST, s_, pb_);                                                     \
      if (live(kb0 + (J) * kBN)) softmax(s_, kb0 + (J) * kBN, pb_);                        \
      issue(desc_k, kb0 + min((J) + 2, ntiles - 1) * kBN, kst(((ST) + 2) & 3));            \
      CPATTN_X8_END_A(J);                                                                  \
    }                                                                                      \
  } while (0)
#define CPATTN_X8_TILE_B(J, ST)                                                            \
  do {                                                                                     \
    if ((J) < ntiles) {                                                                    \
      if ((J) > 0 && live(kb0 + ((J) - 1) * kBN)) softmax(s_, kb0 + ((J) - 1) * kBN, pb_); \
      issue(desc_v, kb0 + min((J) + 2, ntiles - 1) * kBN, vst(((ST) + 2) & 3));            \
      CPATTN_X8_GEMMS(J, ST, s_, pb_);                                                     \
      CPATTN_X8_END_B();                                                                   \
    }                                                                                      \
  } while (0)
  if (wv < 4) {
    for (int j = 0; j < ntiles; j += 4) {
      CPATTN_X8_TILE_A(j, 0);
      CPATTN_X8_TILE_A(j + 1, 1);
      CPATTN_X8_TILE_A(j + 2, 2);
      CPATTN_X8_TILE_A(j + 3, 3);
    }
    // product of the last tile (its stage is not overwritten: the loads
    // issued at the last two tiles went to other stages)
    if (ntiles > 0 && live(kb0 + (ntiles - 1) * kBN)) pv(vst((ntiles - 1) & 3), pb_);
    // the last chunk of the receive
    if constexpr (kRecv)
      if (ntiles > 0) __builtin_nontemporal_store(creg, cdst + chunk_vec(ntiles - 1));
  } else {
    for (int j = 0; j < ntiles; j += 4) {
      // fused ring: the receives of tiles j + 3 .. j + 6, whose loads the
      // waves issue in tiles j + 1 .. j + 4, after the barriers that end
      // tiles j .. j + 3 (tile j + 2's were gated one iteration earlier).
      // Wave 4 polls: in wave 0 the gate cost the loops twelve VGPRs.
      if constexpr (kRing)
        if (wv == 4) gate(kb0 + min(j + 6, ntiles - 1) * kBN);
      CPATTN_X8_TILE_B(j, 0);
      CPATTN_X8_TILE_B(j + 1, 1);
      CPATTN_X8_TILE_B(j + 2, 2);
      CPATTN_X8_TILE_B(j + 3, 3);
    }
    if (ntiles > 0 && live(kb0 + (ntiles - 1) * kBN)) {
      softmax(s_, kb0 + (ntiles - 1) * kBN, pb_);
      pv(vst((ntiles - 1) & 3), pb_);
    }
  }
#undef CPATTN_X8_TILE_B
#undef CPATTN_X8_TILE_A
#undef CPATTN_X8_END_A
#undef CPATTN_X8_END_B
#undef CPATTN_X8_GEMMS

  if (a.tile_cnt && lane == 0) {
    // work counter: the tiles whose scores the loops computed (their
    // condition, live(kb0 + j kBN), over j < ntiles); kept out of the loop,
    // where a counter would cost registers the receive kernel beside this one
    // needs.  kb0 <= w_lo for a wave with rows under document masks.
    const int skipped = kDoc ? max(0, w_lo - kb0) / kBN : 0;
    const int done = max(0, min(ntiles, max(0, (w_max - kb0 + kBN - 1) / kBN)) - skipped);
    __hip_atomic_fetch_add(a.tile_cnt, (unsigned long long)done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  wait_vmem();
  if constexpr (kRecv) {
    // what did not fit in the chunks
    for (int64_t i = rbeg + int64_t(ntiles) * cv + tid; i < rend; i += kThreads8)
      __builtin_nontemporal_store(__builtin_nontemporal_load(csrc + i), cdst + i);
    if (whole_ranges) {
      for (int r = int(blockIdx.x); r < a.recv.n; r += int(gridDim.x)) {
        const g_u32x4* const src = (const g_u32x4*)(a.recv.src[r]);
        g_u32x4* const dst = (g_u32x4*)(a.recv.dst[r]);
        for (int64_t i = tid; i < a.recv.vec[r]; i += kThreads8)
          __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
      }
    }
  }

  l += __shfl_xor(l, 32);
  const int lrow_out = g.q_start + row;
  float lse_s = (m + __builtin_amdgcn_logf(l)) * 0.69314718055994530942f;
  // a row that saw no key (document masks) leaves O_s = 0 and lse_s = -inf
  float inv = kDoc ? (l > 0.f ? 1.f / l : 0.f) : 1.f / l;
  if (ks > 1) {
    // Key split: the part that finishes first leaves its normalised output
    // and LSE in split buffer [part] and exits; the second reads them, folds
    // them into its own by the exact LSE merge and runs the epilogue.  No
    // workgroup waits for another.  The parts travel as device-scope relaxed
    // atomic stores and loads (written through to, and read from, the
    // device's coherence point): a device-scope fence would write back or
    // invalidate the whole L2 of the XCD, under the K/V tiles the other
    // workgroups are still streaming.  The writer's stores have completed
    // (vmcnt 0) before its counter increment; the reader loads only after its
    // increment returned 1.  The merge is symmetric in the two parts, so the
    // result does not depend on which finishes first.
    // Slot of this (row tile, head): the split segments start at a multiple
    // of 256 local rows.  A wave's 16 KiB of the slot hold its lanes' values
    // in register order, chunk k (16 bytes per lane) at k KiB, so every access
    // is a coalesced 1 KiB; the other part's workgroup maps lanes to the same
    // rows and reads the same layout back.  sc1 on the 16-byte buffer
    // accesses: written through to, and read from, device coherence.
    const int64_t slot = int64_t((g.q_start + row0) >> 8) * a.heads + h;
    auto part_rsrc = [&](int pp) {
      return __builtin_amdgcn_make_buffer_rsrc(a.split_o[pp] + (slot * 8 + wv) * 4096, short(0), 16384, 0x00020000);
    };
    constexpr int kSc1 = 16;  // cache-policy operand: sc1 (device scope)
    {
      const __amdgpu_buffer_rsrc_t r = part_rsrc(part);
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          u32x4 v;
#pragma unroll
          for (int u = 0; u < 4; ++u) v[u] = __float_as_uint(__fmul_rn(o[b][4 * q4 + u], inv));
          __builtin_amdgcn_raw_buffer_store_b128(v, r, (4 * b + q4) * 1024 + lane * 16, 0, kSc1);
        }
      if (hf == 0)
        __hip_atomic_store(a.split_lse[part] + slot * 256 + wv * 32 + qc, lse_s, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
    wait_vmem();
    __syncthreads();
    int* const flag = reinterpret_cast<int*>(smem_kv);  // the K/V stages are free by now
    if (tid == 0) {
      int* const cnt = a.split_cnt + slot;
      const int old = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (old != 0) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // ready for the next launch
      *flag = old;
    }
    __syncthreads();
    if (*flag == 0) return;
    if (!ok) return;
    const float lo =
        __hip_atomic_load(a.split_lse[part ^ 1] + slot * 256 + wv * 32 + qc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    float c[NB][16];
    {
      const __amdgpu_buffer_rsrc_t r = part_rsrc(part ^ 1);
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (4 * b + q4) * 1024 + lane * 16, 0, kSc1);
#pragma unroll
          for (int u = 0; u < 4; ++u) c[b][4 * q4 + u] = __uint_as_float(v[u]);
        }
    }
    float w1 = 1.f, w2 = 0.f, L = lse_s;
    if (lo != -INFINITY) {
      if (lse_s == -INFINITY) {
        w1 = 0.f;
        w2 = 1.f;
        L = lo;
      } else {
        L = fmaxf(lse_s, lo) + log1pf(expf(-fabsf(lse_s - lo)));
        w1 = expf(lse_s - L);
        w2 = expf(lo - L);
      }
    }
    // both terms exactly as the other order would form them: own value
    // rounded as it would have been stored, products and sum rounded one by
    // one (no contraction), a term of weight 0 left out
    auto mix = [&](float own, float other) {
      const float t1 = w1 != 0.f ? __fmul_rn(w1, __fmul_rn(own, inv)) : 0.f;
      const float t2 = w2 != 0.f ? __fmul_rn(w2, other) : 0.f;
      return __fadd_rn(t1, t2);
    };
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[b][e] = mix(o[b][e], c[b][e]);
    lse_s = L;
    inv = 1.f;
  }
  if (!ok) return;
  // document masks: a row that saw no key leaves a merge-only step's running
  // state as it is
  if (kDoc && l == 0.f && epi == kEpiMerge) return;
  float4 c[NB][4];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) c[b][q4] = row_epi_load4(a, epi, h, lrow_out, 32 * b + 8 * q4 + 4 * hf, D);
  const RowEpi e = row_epi_begin(a, epi, h, lrow_out, lse_s);
#pragma unroll
  for (int b = 0; b < NB; ++b) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const float4 v4 = make_float4(o[b][4 * q4] * inv, o[b][4 * q4 + 1] * inv, o[b][4 * q4 + 2] * inv,
                                    o[b][4 * q4 + 3] * inv);
      row_epi_store4(a, epi, e, h, lrow_out, grow, 32 * b + 8 * q4 + 4 * hf, D, v4, c[b][q4]);
    }
  }
  if (hf == 0) row_epi_store_lse(a, epi, e, h, lrow_out, grow, lse_s);
}

}  // namespace

int attn_bf16_block_m(int head_dim) { return head_dim == 128 ? kBM8 : kBM; }

bool attn_does_recv(int dtype_bf16, int head_dim) { return dtype_bf16 && head_dim == 128; }

bool attn_splits_keys(int dtype_bf16, int head_dim) { return dtype_bf16 && head_dim == 128; }

hipError_t launch_attn_bf16_ranks(const StepArgs* tbl, const int32_t* wgb, int nranks, int total_wgs, bool doc,
                                  hipStream_t stream) {
  if (total_wgs <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(total_wgs));
  if (doc)
    attn_step_bf16_d128x8<false, true, true><<<grid, kThreads8, 0, stream>>>(StepArgs{}, tbl, wgb, nranks);
  else
    attn_step_bf16_d128x8<false, false, true><<<grid, kThreads8, 0, stream>>>(StepArgs{}, tbl, wgb, nranks);
  return hipGetLastError();
}

hipError_t launch_attn_bf16_ring(const StepArgs& a, hipStream_t stream) {
  const dim3 grid(unsigned(a.total_tiles) * unsigned(a.heads));
  attn_step_bf16_d128x8<false, false, false, true><<<grid, kThreads8, 0, stream>>>(a, nullptr, nullptr, 0);
  return hipGetLastError();
}

hipError_t launch_attn_bf16(const StepArgs& a, int head_dim, hipStream_t stream) {
  const dim3 grid(unsigned(a.total_tiles) * unsigned(a.heads));
  if (head_dim == 128) {
    if (a.doc) {
      if (a.recv.n > 0)
        attn_step_bf16_d128x8<true, true, false><<<grid, kThreads8, 0, stream>>>(a, nullptr, nullptr, 0);
      else
        attn_step_bf16_d128x8<false, true, false><<<grid, kThreads8, 0, stream>>>(a, nullptr, nullptr, 0);
    } else if (a.recv.n > 0) {
      attn_step_bf16_d128x8<true, false, false><<<grid, kThreads8, 0, stream>>>(a, nullptr, nullptr, 0);
    } else {
      attn_step_bf16_d128x8<false, false, false><<<grid, kThreads8, 0, stream>>>(a, nullptr, nullptr, 0);
    }
  } else {
    attn_step_bf16<64><<<grid, kThreads, 0, stream>>>(a);
  }
  return hipGetLastError();
}

}  // namespace cpattn
