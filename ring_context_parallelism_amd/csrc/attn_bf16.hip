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
//   * workgroup = 4 waves = 128 query rows of one head; wave w owns 32 rows.
//   * scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16: A = K from LDS (row = key), B = Q^T from
//     registers (column = query).  The 32x32 result leaves every lane with 16
//     keys of ONE query, so the row max and row sum are per-lane reductions
//     plus a single exchange with the lane 32 away.
//   * O^T = V^T P^T with the same instruction: B = P^T straight from the score
//     registers (converted to bf16, round-to-nearest-even), A = V^T from LDS.
//     V is transposed on its way into LDS and, within every 16-key group, the
//     key order is permuted to match the order in which the score registers
//     hold keys, so P never leaves registers.
//   * K/V tiles of 64 keys are fetched with buffer loads (hardware range
//     check: keys past the slot read as zero) two tiles ahead into registers,
//     then written to a double-buffered LDS tile (K row-major, V transposed);
//     16-byte padded rows keep the matrix-operand reads bank-conflict free and
//     the transposed V writes are spread over distinct banks.
//   * softmax in base 2: p = exp2(s * scale * log2 e - m); the reference max m
//     is only raised when a tile's max exceeds it by more than 8 (p <= 2^8 in
//     between), which skips most O rescales and is exact for any choice of m.
//   * workgroup ids are remapped so consecutive logical tiles (same head, same
//     K/V) share an XCD and its L2; the logical order puts the longest rows of
//     a diagonal segment first.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "epilogue.h"
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

  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int h = L / a.total_tiles;
  int t = L % a.total_tiles;
  const int si = t < a.seg[0].tiles ? 0 : 1;
  if (si) t -= a.seg[0].tiles;
  const SegArgs& g = a.seg[si];
  if (g.diag) t = g.tiles - 1 - t;  // longest rows first
  const int row0 = t * kBM;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int qc = lane & 31, hf = lane >> 5;
  const int row = row0 + wv * 32 + qc;  // row within the segment
  const bool ok = row < g.q_len;

  const int tile_last = min(row0 + kBM, g.q_len);
  const int kv_end = g.kv_full + (g.diag ? tile_last : 0);
  const int w_first = row0 + wv * 32;
  const int w_last = min(w_first + 32, g.q_len);
  const bool w_active = w_last > w_first;
  const int w_max = w_active ? g.kv_full + (g.diag ? w_last : 0) : 0;      // longest prefix in the wave
  const int w_min = g.kv_full + (g.diag ? w_first + 1 : 0);                // shortest prefix in the wave
  const int prefix = ok ? g.kv_full + (g.diag ? row + 1 : 0) : w_max;

  const int64_t hd = int64_t(a.heads) * D;
  const int64_t grow = g.q_global + row;

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

  // K/V slot reads go through buffer resources: a key past the slot's last
  // row is outside num_records and loads as zero (and is masked anyway).
  const uint32_t row_bytes = uint32_t(a.heads) * D * 2;
  const uint32_t slot_bytes = uint32_t(a.n_loc) * row_bytes;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.k, slot_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(a.v, slot_bytes);
  const uint32_t head_off = uint32_t(h) * D * 2;

  u32x4 kreg[KCH];
  u32x4 vreg[4];
  // V item of this thread: keys 4 vkg .. 4 vkg + 3, dims 8 vdg .. 8 vdg + 7.
  // Sixteen consecutive lanes take sixteen key groups of one dim group, so
  // their 8-byte transposed writes land on sixteen different bank pairs.
  const int vkg = tid & 15, vdg = tid >> 4;

  auto load_tile = [&](int j0) {
    const uint32_t base = uint32_t(j0) * row_bytes + head_off;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = tid + kThreads * i;
      const int kr = c / CPR, cc = c % CPR;
      kreg[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, base + uint32_t(kr) * row_bytes + cc * 16, 0, 0);
    }
    if (tid < VITEMS) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        vreg[e] = __builtin_amdgcn_raw_buffer_load_b128(rv, base + uint32_t(4 * vkg + e) * row_bytes + vdg * 16, 0, 0);
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
  const int ntiles = (kv_end + kBN - 1) / kBN;
  if (ntiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  if (ntiles > 1) load_tile(kBN);
  __syncthreads();
  for (int it = 0; it < ntiles; ++it) {
    const int j0 = it * kBN;
    const int buf = it & 1;
    if (j0 < w_max) {
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
      if (j0 + kBN > w_min) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = j0 + 32 * kb + 8 * (i >> 2) + 4 * hf + (i & 3);
            if (key >= prefix) s[kb][i] = -INFINITY;
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
      if (it + 2 < ntiles) load_tile((it + 2) * kBN);
    }
    __syncthreads();
  }

  l += __shfl_xor(l, 32);
  if (!ok) return;
  const int lrow = g.q_start + row;
  const float lse_s = (m + __builtin_amdgcn_logf(l)) * 0.69314718055994530942f;
  const float inv = 1.f / l;
  const RowEpi e = row_epi_begin(a, g, h, lrow, lse_s);
#pragma unroll
  for (int b = 0; b < NB; ++b) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const float4 v4 = make_float4(o[b][4 * q4] * inv, o[b][4 * q4 + 1] * inv, o[b][4 * q4 + 2] * inv,
                                    o[b][4 * q4 + 3] * inv);
      row_epi_store4(a, g, e, h, lrow, grow, 32 * b + 8 * q4 + 4 * hf, D, v4);
    }
  }
  if (hf == 0) row_epi_store_lse(a, g, e, h, lrow, grow, lse_s);
}

}  // namespace

int attn_bf16_block_m() { return kBM; }

hipError_t launch_attn_bf16(const StepArgs& a, int head_dim, hipStream_t stream) {
  const dim3 grid(unsigned(a.total_tiles) * unsigned(a.heads));
  if (head_dim == 128) {
    attn_step_bf16<128><<<grid, kThreads, 0, stream>>>(a);
  } else {
    attn_step_bf16<64><<<grid, kThreads, 0, stream>>>(a);
  }
  return hipGetLastError();
}

}  // namespace cpattn
