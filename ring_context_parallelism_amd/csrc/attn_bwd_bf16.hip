// Backward of one ring step on gfx950 matrix cores: bf16, head_dim 128.
//
// The same step and the same terms as the generic kernels in attn_bwd.hip
// (gradients of the step's valid pairs with the complete forward's LSE and
// D_i = <dO_i, O_i>; "Context Parallelism for Long-Context Training", section
// "Prove attention equivalence"; valid pairs and skipped future sub-blocks as
// in "Sequence Parallelism IV: Megatron Context Parallel and Load-Balanced
// Rings", section 4), with every product on v_mfma_f32_32x32x16_bf16:
//
// Key-major kernel (dK, dV): a workgroup of 4 waves owns 128 keys of one head,
// 32 per wave, whose K and V rows stay in registers as the B operand
// (column = key).  Tiles of 64 of the rank's rows (Q and dO, row-major with
// the XOR swizzle of the forward's K/V tiles) are staged in LDS:
//   S = Q K^T and dP = dO V^T   (A = Q / dO rows from LDS; lane = one key)
//   P = exp2(S scale log2e - LSE log2e), dS = P (dP - D)   (per element)
//   dV^T += dO^T P and dK^T += Q^T dS   (A = dO^T / Q^T read transposed
//   from the same tiles with ds_read_b64_tr_b16; B = P / dS straight from
//   the registers of S, rounded to bf16, rows in register order)
// Row-major kernel (dQ): a workgroup of 8 waves owns 256 rows, 32 per wave,
// whose Q and dO stay in registers; K/V tiles of 64 keys stream into LDS:
//   S^T = K Q^T, dP^T = V dO^T, dS^T as above, dQ^T += K^T dS^T.
// Rows past a segment's end carry LSE = +inf, so their P is exactly zero;
// keys past the source's real keys are clamped to its last real row and
// masked.  The key-major kernel loads its tiles to registers one tile ahead
// and stores them to LDS after the barrier that ends the previous tile.
//
// Document masks: every row sees only its document's run of the source's
// keys, [klo, khi).  The rows of a segment are consecutive positions, so klo
// and khi grow with the row: the key-major kernel skips a row tile whose runs
// miss the wave's keys and stops at the first tile that starts past its
// keys; the row-major kernel starts at its first row's run.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>

#include "epilogue.h"
#include "kernels.h"
#include "lds_dma.h"

namespace cpattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

constexpr int D = 128;
constexpr int NT = D / 16;     // k-steps over the head dimension
constexpr int NB = D / 32;     // 32-row blocks of a transposed gradient
constexpr int kThreads = 256;  // 4 waves
constexpr int kKeys = 128;     // keys per key-major workgroup (32 per wave)
constexpr int kTileRows = 64;  // rows of an LDS tile (Q/dO rows or K/V keys)
constexpr int kTileBytes = kTileRows * 256;
constexpr float kLog2e = 1.4426950408889634f;

// Permutation of the 16 16-byte chunks of a 256-byte tile row (linear over
// GF(2) in the row's low four bits); logical chunk c of row r is stored at
// chunk c ^ swz(r & 15), so that the operand reads below hit distinct banks.
__device__ __forceinline__ int swz(int r) {
  return ((r >> 2) & 1) | ((((r >> 1) ^ (r >> 3)) & 1) << 1) | ((r & 1) << 2) | (((r >> 1) & 1) << 3);
}

__device__ __forceinline__ int kv_row(const BwdArgs& a, int kk) {
  return kk < a.kv_split ? a.kv_lo + kk : a.kv_hi + (kk - a.kv_split);
}

// Per-lane LDS offsets of the operand reads (see the forward's tiles):
//   row reads: lane (row qc, half hf) takes logical chunk 2 i + hf of row qc
//   transposed reads: lane (group g1, index i16) points at row 8 r + 4 hf +
//   i16/4 of a 16-row group, bytes 32 g1 + 8 (i16 & 3) .. + 7 of a 64-byte block
struct Bases {
  uint32_t row;
  uint32_t tr[2];
};

__device__ __forceinline__ Bases make_bases(int lane) {
  const int qc = lane & 31, hf = lane >> 5;
  Bases b;
  b.row = qc * 256 + ((hf ^ swz(qc & 15)) << 4);
  const int i16 = lane & 15, g1 = (lane >> 4) & 1;
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int vr = 8 * r + 4 * hf + (i16 >> 2);
    const int c0 = 2 * g1 + ((i16 & 3) >> 1);
    b.tr[r] = vr * 256 + ((c0 ^ swz(vr & 15)) << 4) + 8 * (i16 & 1);
  }
  return b;
}

// C[row][col] over two 32-row blocks of a 64-row tile: A = tile rows (LDS),
// B = the lane's resident column operand (8 k-steps over the head dimension).
__device__ __forceinline__ void mm_rows(const lds_u8* tile, uint32_t base, const bf16x8 (&b)[NT], f32x16 (&c)[2]) {
  c[0] = f32x16{};
  c[1] = f32x16{};
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const bf16x8 a0 = *reinterpret_cast<const lds_bf16x8*>(tile + (base ^ (32u * i)));
    const bf16x8 a1 = *reinterpret_cast<const lds_bf16x8*>(tile + 32 * 256 + (base ^ (32u * i)));
    c[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b[i], c[0], 0, 0, 0);
    c[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b[i], c[1], 0, 0, 0);
  }
}

// acc^T[d][col] += sum over the tile's 64 rows of tile[row][d] * w[row][col]:
// A = the tile read transposed, B = w from registers (rows in register order).
__device__ __forceinline__ void mm_tr(const lds_u8* tile, const uint32_t (&tr)[2], const bf16x8 (&w)[2][2],
                                      f32x16 (&acc)[NB]) {
#pragma unroll
  for (int gq = 0; gq < 4; ++gq) {
    const int kb = gq >> 1, u = gq & 1;
    const int roff = (32 * kb + 16 * u) * 256;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + roff + (tr[0] ^ (64u * b))));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + roff + (tr[1] ^ (64u * b))));
      const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, w[kb][u], acc[b], 0, 0, 0);
    }
  }
}

// 64 rows x 256 bytes from global (row r at src_row(r) * row_bytes + hoff)
// into registers, four 16-byte chunks per thread; then into a swizzled tile.
struct TileRegs {
  u32x4 x[4];
};

template <typename RowFn>
__device__ __forceinline__ void tile_load(TileRegs& t, const void* base, uint32_t row_bytes, uint32_t hoff, int tid,
                                          RowFn src_row) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + kThreads * i;
    const int r = c >> 4, ch = c & 15;
    const char* p = static_cast<const char*>(base) + uint64_t(src_row(r)) * row_bytes + hoff + ch * 16;
    t.x[i] = *reinterpret_cast<const u32x4*>(p);
  }
}

__device__ __forceinline__ void tile_store(const TileRegs& t, lds_u8* tile, int tid) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + kThreads * i;
    const int r = c >> 4, ch = c & 15;
    *reinterpret_cast<lds_u32x4*>(tile + r * 256 + ((ch ^ swz(r & 15)) << 4)) = t.x[i];
  }
}

// ---------------------------------------------------------------------------
// Key-major: dK and dV of 128 keys.
// ---------------------------------------------------------------------------
template <bool kDoc>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(1, 1)))
void bwd_dkdv_bf16_d128(BwdArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * kTileBytes];
  __shared__ __attribute__((aligned(16))) float s_lse[kTileRows];
  __shared__ __attribute__((aligned(16))) float s_del[kTileRows];
  __shared__ __attribute__((aligned(16))) int s_klo[kTileRows];  // document masks: the rows' key runs
  __shared__ __attribute__((aligned(16))) int s_khi[kTileRows];
  lds_u8* const tq = (lds_u8*)smem;
  lds_u8* const tdo = tq + kTileBytes;

  const int h = blockIdx.x % a.heads;
  const int k0 = (blockIdx.x / a.heads) * kKeys;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qc = lane & 31, hf = lane >> 5;
  const int key = k0 + 32 * wv + qc;
  const bool kok = key < a.kv_valid;
  const int krow = kv_row(a, min(key, a.kv_valid - 1));
  const uint32_t row_bytes = uint32_t(a.heads) * 256;
  const uint32_t hoff = uint32_t(h) * 256;

  bf16x8 kf[NT], vf[NT];
  {
    const __bf16* kp = static_cast<const __bf16*>(a.k) + (int64_t(krow) * a.heads + h) * D + 8 * hf;
    const __bf16* vp = static_cast<const __bf16*>(a.v) + (int64_t(krow) * a.heads + h) * D + 8 * hf;
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      kf[i] = *reinterpret_cast<const bf16x8*>(kp + 16 * i);
      vf[i] = *reinterpret_cast<const bf16x8*>(vp + 16 * i);
    }
  }
  f32x16 dk[NB], dv[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    dk[b] = f32x16{};
    dv[b] = f32x16{};
  }
  const Bases bs = make_bases(lane);
  const int w_key0 = k0 + 32 * wv;  // the wave's smallest key

  for (int si = 0; si < a.nseg; ++si) {
    const SegArgs& g = a.seg[si];
    int t0;
    if (k0 < g.kv_full) t0 = 0;
    else if (g.diag) t0 = k0 - g.kv_full;  // row t sees keys < kv_full + t + 1
    else continue;
    if (t0 >= g.q_len) continue;
    auto qrow = [&](int r) { return g.q_global + min(r, g.q_len - 1); };
    TileRegs rq, rdo;
    tile_load(rq, a.q, row_bytes, hoff, tid, [&](int r) { return qrow(t0 + r); });
    tile_load(rdo, a.dout, row_bytes, hoff, tid, [&](int r) { return qrow(t0 + r); });
    for (int r0 = t0; r0 < g.q_len; r0 += kTileRows) {
      __syncthreads();  // the previous tile's reads are done
      tile_store(rq, tq, tid);
      tile_store(rdo, tdo, tid);
      if (tid < kTileRows) {
        const int t = r0 + tid;
        const bool ok = t < g.q_len;
        s_lse[tid] = ok ? a.lse[int64_t(h) * a.seq_len + g.q_global + t] * kLog2e : INFINITY;
        s_del[tid] = ok ? a.delta[int64_t(h) * a.n_loc + g.q_start + t] : 0.f;
        if constexpr (kDoc) {
          int lo, hi;
          doc_row_keys(a, qrow(t), lo, hi);
          s_klo[tid] = lo;
          s_khi[tid] = hi;
        }
      }
      __syncthreads();
      // document masks: runs start no earlier than the tile's first row's, end
      // no later than its last row's; no later tile reaches these keys once
      // a tile's first run starts past them
      int tile_klo = 0, tile_khi = 0x7fffffff;  // (no document bound)
      if constexpr (kDoc) {
        tile_klo = s_klo[0];
        tile_khi = s_khi[min(kTileRows, g.q_len - r0) - 1];
        if (tile_klo >= k0 + kKeys) break;
      }
      if (r0 + kTileRows < g.q_len) {  // next tile in flight during this one
        tile_load(rq, a.q, row_bytes, hoff, tid, [&](int r) { return qrow(r0 + kTileRows + r); });
        tile_load(rdo, a.dout, row_bytes, hoff, tid, [&](int r) { return qrow(r0 + kTileRows + r); });
      }
      // the wave's keys against the tile's longest prefix
      const int tile_pre = g.kv_full + (g.diag ? min(r0 + kTileRows, g.q_len) : 0);
      if (w_key0 >= min(tile_pre, tile_khi) || (kDoc && w_key0 + 32 <= tile_klo)) continue;
      f32x16 s[2], dp[2];
      mm_rows(tq, bs.row, kf, s);
      mm_rows(tdo, bs.row, vf, dp);
      bf16x8 wp[2][2], ws[2][2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int rl = 32 * qb + 8 * m + 4 * hf;  // tile row of register 4 m
          const float4 l4 = *reinterpret_cast<const float4*>(&s_lse[rl]);
          const float4 d4 = *reinterpret_cast<const float4*>(&s_del[rl]);
          const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
          const float dl[4] = {d4.x, d4.y, d4.z, d4.w};
          int klo[4] = {0, 0, 0, 0}, khi[4] = {a.n_loc, a.n_loc, a.n_loc, a.n_loc};
          if constexpr (kDoc) {
            const int4 lo4 = *reinterpret_cast<const int4*>(&s_klo[rl]);
            const int4 hi4 = *reinterpret_cast<const int4*>(&s_khi[rl]);
            klo[0] = lo4.x, klo[1] = lo4.y, klo[2] = lo4.z, klo[3] = lo4.w;
            khi[0] = hi4.x, khi[1] = hi4.y, khi[2] = hi4.z, khi[3] = hi4.w;
          }
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int e = 4 * m + c;
            const int t = r0 + rl + c;
            const int pre = kDoc ? min(g.kv_full + (g.diag ? t + 1 : 0), khi[c]) : g.kv_full + (g.diag ? t + 1 : 0);
            const float p = key < pre && (!kDoc || key >= klo[c])
                                ? __builtin_amdgcn_exp2f(fmaf(s[qb][e], a.scale_log2, -lv[c]))
                                : 0.f;
            const float ds = p * (dp[qb][e] - dl[c]);
            wp[qb][e >> 3][e & 7] = static_cast<__bf16>(p);
            ws[qb][e >> 3][e & 7] = static_cast<__bf16>(ds);
          }
        }
      }
      mm_tr(tdo, bs.tr, wp, dv);
      mm_tr(tq, bs.tr, ws, dk);
    }
  }
  if (!kok) return;
  // lane (key, hf) holds d = 32 b + 8 m + 4 hf + c of its key
  float* dkp = a.dk + (int64_t(krow) * a.heads + h) * D;
  float* dvp = a.dv + (int64_t(krow) * a.heads + h) * D;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int d0 = 32 * b + 8 * m + 4 * hf;
      float4 x = *reinterpret_cast<float4*>(dkp + d0);
      float4 y = *reinterpret_cast<float4*>(dvp + d0);
      x.x += a.scale * dk[b][4 * m + 0];
      x.y += a.scale * dk[b][4 * m + 1];
      x.z += a.scale * dk[b][4 * m + 2];
      x.w += a.scale * dk[b][4 * m + 3];
      y.x += dv[b][4 * m + 0];
      y.y += dv[b][4 * m + 1];
      y.z += dv[b][4 * m + 2];
      y.w += dv[b][4 * m + 3];
      *reinterpret_cast<float4*>(dkp + d0) = x;
      *reinterpret_cast<float4*>(dvp + d0) = y;
    }
  }
}

// ---------------------------------------------------------------------------
// Key-major, eight waves: the same products as above with the work of a
// 32-key column split between two waves of one SIMD.
// ---------------------------------------------------------------------------
// Waves w and w + 4 (on one SIMD) own keys 32 (w & 3) .. + 31 of the
// workgroup's 128.  Wave w (S role) holds K, computes S = Q K^T and P and
// accumulates dV; wave w + 4 (dP role) holds V, computes dP = dO V^T, takes
// P (fp32) through LDS, forms dS and accumulates dK.  Each wave then needs
// one K or V operand and one 32x128 accumulator, half the registers of the
// one-pass kernel, so two waves share a SIMD.  The dP role runs one tile
// behind: with tiles T_0 .. T_{n-1}, phase p is
//   [X_p .. Y_p]   S role: dV += dO(T_{p-1})^T P, S(T_p)     (32 MFMAs)
//                  dP role: dS(T_{p-1}) = P (dP - D)        (vector ALU)
//   [Y_p .. X_p+1] S role: P(T_p) from S(T_p), to LDS       (vector ALU)
//                  dP role: dK += Q(T_{p-1})^T dS, dP(T_p)  (32 MFMAs)
// between workgroup barriers X and Y, so on every SIMD one wave's matrix
// work runs while the other's elementwise work does.  Phase p reads the tile
// stages of T_p and T_{p-1} and fills the third with T_{p+1}, loaded to
// registers at the phase's start.  Per wave the products, their operands and
// the order over tiles are those of the one-pass kernel: dK and dV are
// bit-identical to it.
constexpr int kThreads8 = 512;
constexpr int kStages = 3;

// mm_rows with the operand reads two k-steps ahead of the MFMAs (pinned by
// scheduling-group barriers): one wave issues the reads and MFMAs of a
// product alone, so the LDS latency has to hide behind its own MFMAs.
__device__ __forceinline__ void mm_rows_p(const lds_u8* tile, uint32_t base, const bf16x8 (&b)[NT], f32x16 (&c)[2]) {
  bf16x8 a0[NT], a1[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    a0[i] = *reinterpret_cast<const lds_bf16x8*>(tile + (base ^ (32u * i)));
    a1[i] = *reinterpret_cast<const lds_bf16x8*>(tile + 32 * 256 + (base ^ (32u * i)));
  }
  c[0] = f32x16{};
  c[1] = f32x16{};
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    c[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0[i], b[i], c[0], 0, 0, 0);
    c[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1[i], b[i], c[1], 0, 0, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // k-steps 0, 1 read
#pragma unroll
  for (int i = 0; i < NT - 2; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // k-step i
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // k-step i + 2 read
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);  // k-steps NT - 2, NT - 1
}

// mm_tr with the transposed reads one group of four MFMAs ahead.
__device__ __forceinline__ void mm_tr_p(const lds_u8* tile, const uint32_t (&tr)[2], const bf16x8 (&w)[2][2],
                                        f32x16 (&acc)[NB]) {
  bf16x8 va[4][NB];
#pragma unroll
  for (int gq = 0; gq < 4; ++gq) {
    const int roff = (32 * (gq >> 1) + 16 * (gq & 1)) * 256;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + roff + (tr[0] ^ (64u * b))));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + roff + (tr[1] ^ (64u * b))));
      va[gq][b] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  }
#pragma unroll
  for (int gq = 0; gq < 4; ++gq)
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[gq][b], w[gq >> 1][gq & 1], acc[b], 0, 0, 0);
  __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);  // groups 0 and 1 read
  __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);   // group 0 MFMAs
  __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);   // group 2 read
  __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);   // group 1 MFMAs
  __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);   // group 3 read
  __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);   // groups 2 and 3 MFMAs
}

// Workgroup barrier that orders LDS accesses only: global and direct-to-LDS
// loads in flight stay in flight across it (a wave waits for its own
// direct-to-LDS loads with vmcnt before the barrier that publishes them).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Segment si of the step (0 or 1) by field-wise selection from two copies
// held in scalar registers: no indexed load of the kernel arguments inside
// the tile loop (a chain of dependent scalar loads each phase).
__device__ __forceinline__ SegArgs seg_pick(const SegArgs& x, const SegArgs& y, int si) {
  SegArgs r;
  r.q_global = si ? y.q_global : x.q_global;
  r.q_start = si ? y.q_start : x.q_start;
  r.q_len = si ? y.q_len : x.q_len;
  r.kv_full = si ? y.kv_full : x.kv_full;
  r.diag = si ? y.diag : x.diag;
  r.epi = si ? y.epi : x.epi;
  r.tiles = si ? y.tiles : x.tiles;
  r.ksplit = si ? y.ksplit : x.ksplit;
  return r;
}

// The next 64-row tile of a key-major workgroup's walk (keys k0 .. k0 + 127):
// the search starts at row r0 of segment si (r0 < 0: the segment's first
// tile).  Rows before a segment's first tile see none of the keys; with
// document masks the walk leaves a segment at the first tile whose first
// row's run starts past them.  Leaves si = nseg when no tile is left.  One
// exit, at the loop's end.
template <bool kDoc>
__device__ __forceinline__ void km_seek(const BwdArgs& a, const SegArgs& s0, const SegArgs& s1, int k0, int& si,
                                        int& r0) {
  bool found = false;
  while (!found && si < a.nseg) {
    const SegArgs g = seg_pick(s0, s1, si);
    // row t sees keys < kv_full + t + 1 on a diagonal segment
    const int t0 = k0 < g.kv_full ? 0 : (g.diag ? k0 - g.kv_full : g.q_len);
    if (r0 < 0) r0 = t0;
    found = r0 < g.q_len;
    if constexpr (kDoc) {
      if (found) {
        int lo, hi;
        doc_row_keys(a, g.q_global + r0, lo, hi);
        found = lo < k0 + kKeys;
      }
    }
    if (!found) {
      ++si;
      r0 = -1;
    }
  }
}

// Per-row tables of one tile, loaded by wave 0 (a lane per row) one phase
// ahead: raw LSE and D (rows at or past `rows` are replaced when stored),
// and the rows' document runs.
struct KmRows {
  float lse, del;
  int rows;
  int klo, khi;
};

template <bool kDoc>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads8, kThreads8), amdgpu_waves_per_eu(2, 2)))
void bwd_dkdv_bf16_d128x8(BwdArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kStages * 2 * kTileBytes];
  __shared__ __attribute__((aligned(16))) float s_p[4 * 2 * 4 * 64 * 4];  // P of each wave pair, fp32
  __shared__ __attribute__((aligned(16))) float s_lse[kStages][kTileRows];
  __shared__ __attribute__((aligned(16))) float s_del[kStages][kTileRows];
  __shared__ __attribute__((aligned(16))) int s_klo[kStages][kTileRows];
  __shared__ __attribute__((aligned(16))) int s_khi[kStages][kTileRows];

  const int h = blockIdx.x % a.heads;
  const int k0 = (blockIdx.x / a.heads) * kKeys;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int role = wv >> 2, pw = wv & 3;  // role 0: S, P, dV; role 1: dP, dS, dK
  const int qc = lane & 31, hf = lane >> 5;
  const int w_key0 = k0 + 32 * pw;  // the pair's smallest key
  const int key = w_key0 + qc;
  const bool kok = key < a.kv_valid;
  const int krow = kv_row(a, min(key, a.kv_valid - 1));
  const uint32_t row_bytes = uint32_t(a.heads) * 256;
  const uint32_t hoff = uint32_t(h) * 256;
  const Bases bs = make_bases(lane);
  float* const pbuf = s_p + pw * (2 * 4 * 64 * 4) + lane * 4;  // + (4 qb + m) * 256: float4 of the lane
  const SegArgs sg0 = a.seg[0], sg1 = a.seg[1];

  auto stage_q = [&](int st) { return (lds_u8*)smem + st * 2 * kTileBytes; };
  auto stage_o = [&](int st) { return (lds_u8*)smem + st * 2 * kTileBytes + kTileBytes; };

  // Tile loads straight into LDS: 32 loads of 1 KiB per tile (Q, then dO,
  // four rows each: lane = row 4 b + lane / 16 of block b, physical chunk
  // lane % 16, which holds logical chunk (lane % 16) ^ swz(row)).  Pair pw
  // issues loads 8 pw .. 8 pw + 7 (Q for pairs 0-1, dO for pairs 2-3): its
  // S-role wave the first two, during its P work, its dP-role wave the other
  // six, during its dS work (which is shorter than the other wave's matrix
  // work, while P is not).  Offsets are 32-bit, from a base at each
  // segment's first row (a segment spans at most the rank's rows, which the
  // plan keeps below 4 GiB).
  const char* const dma_src = static_cast<const char*>(pw < 2 ? a.q : a.dout);
  const dma_u32x4 desc0 = buffer_desc(dma_src + uint64_t(sg0.q_global) * row_bytes, uint32_t(sg0.q_len) * row_bytes);
  const dma_u32x4 desc1 = buffer_desc(dma_src + uint64_t(sg1.q_global) * row_bytes, uint32_t(sg1.q_len) * row_bytes);
  const int dma_r = 32 * (pw & 1) + (lane >> 4);  // + 4 j: the lane's tile row for load 8 pw + j
  uint32_t dma_c[4];  // + row * row_bytes: the lane's global byte offset (depends on j mod 4)
#pragma unroll
  for (int j = 0; j < 4; ++j) dma_c[j] = uint32_t(((lane & 15) ^ swz((dma_r + 4 * j) & 15)) << 4) + hoff;
  auto issue_loads = [&](int si, int r0, int st, auto j0, auto j1) {
    const SegArgs g = seg_pick(sg0, sg1, si);
    const dma_u32x4 desc = si ? desc1 : desc0;
    const uint32_t dst = lds_addr((pw < 2 ? stage_q(st) : stage_o(st)) + 32 * (pw & 1) * 256);
#pragma unroll
    for (int j = decltype(j0)::value; j < decltype(j1)::value; ++j) {
      const int row = min(r0 + dma_r + 4 * j, g.q_len - 1);  // of the segment
      // 24-bit multiply: row and row_bytes are below 2^24 and their product
      // below 2^32 (a 64-bit multiply-add here reads an undefined high half
      // that can alias a register with a load in flight, and then waits for it)
      dma_lds16(desc, __umul24(uint32_t(row), row_bytes) + dma_c[j & 3], 0u, dst + j * 1024);
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I2 = std::integral_constant<int, 2>;
  using I8 = std::integral_constant<int, 8>;
  auto issue_tile = [&](int si, int r0, int st) { issue_loads(si, r0, st, I0{}, I8{}); };  // prologue
  auto load_rows = [&](int si, int r0, KmRows& rg) {  // wave 0
    const SegArgs g = seg_pick(sg0, sg1, si);
    const int tc = min(r0 + lane, g.q_len - 1);
    rg.lse = a.lse[int64_t(h) * a.seq_len + g.q_global + tc];
    rg.del = a.delta[int64_t(h) * a.n_loc + g.q_start + tc];
    rg.rows = g.q_len - r0;
    if constexpr (kDoc) doc_row_keys(a, g.q_global + tc, rg.klo, rg.khi);
  };
  // wave 0; rows past the segment: LSE = +inf (P = 0), D = 0
  auto store_rows = [&](int st, const KmRows& rg) {
    const bool ok = lane < rg.rows;
    s_lse[st][lane] = ok ? rg.lse * kLog2e : INFINITY;
    s_del[st][lane] = ok ? rg.del : 0.f;
    if constexpr (kDoc) {
      s_klo[st][lane] = rg.klo;
      s_khi[st][lane] = rg.khi;
    }
  };
  // does the pair have a valid pair in tile (si, r0), held in stage st?
  auto pair_active = [&](int si, int r0, int st) {
    const SegArgs g = seg_pick(sg0, sg1, si);
    const int tile_pre = g.kv_full + (g.diag ? min(r0 + kTileRows, g.q_len) : 0);
    if constexpr (kDoc) {
      const int tile_klo = s_klo[st][0];
      const int tile_khi = s_khi[st][min(kTileRows, g.q_len - r0) - 1];
      return !(w_key0 >= min(tile_pre, tile_khi) || w_key0 + 32 <= tile_klo);
    }
    return w_key0 < tile_pre;
  };

  bf16x8 kv[NT];  // K (S role) or V (dP role) of the lane's key
  {
    const void* src = role == 0 ? a.k : a.v;
    const __bf16* p = static_cast<const __bf16*>(src) + (int64_t(krow) * a.heads + h) * D + 8 * hf;
#pragma unroll
    for (int i = 0; i < NT; ++i) kv[i] = *reinterpret_cast<const bf16x8*>(p + 16 * i);
  }
  f32x16 acc[NB];  // dV^T (S role) or dK^T (dP role)
#pragma unroll
  for (int b = 0; b < NB; ++b) acc[b] = f32x16{};

  int c_si = 0, c_r0 = -1;
  km_seek<kDoc>(a, sg0, sg1, k0, c_si, c_r0);
  bool c_ok = c_si < a.nseg;  // T_p exists
  KmRows rg{};
  if (c_ok) {
    if (role == 0) issue_tile(c_si, c_r0, 0);  // the S-role waves load T_0 alone
    if (wv == 0) {
      load_rows(c_si, c_r0, rg);
      store_rows(0, rg);
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the K/V rows above and this wave's tile loads
  lds_barrier();                       // X_0
  bool p_act = false;  // T_{p-1} exists and has work for the pair
  int st = 0;          // stage of T_p; T_{p-1} in (st + 2) % 3, T_{p+1} goes to (st + 1) % 3
  auto next_tile = [&](int& n_si, int& n_r0, bool& n_ok) {
    n_si = c_si;
    n_r0 = c_r0 + kTileRows;
    n_ok = false;
    if (c_ok) {
      km_seek<kDoc>(a, sg0, sg1, k0, n_si, n_r0);
      n_ok = n_si < a.nseg;
      if (n_ok && wv == 0) load_rows(n_si, n_r0, rg);
    }
  };
  // End of phase p: the next tile's row tables, wait for this wave's loads
  // of T_{p+1}, barrier X_{p+1}, advance.  Returns false after phase n
  // (T_{n-1} was the last tile).
  auto end_phase = [&](int n_si, int n_r0, bool n_ok, bool c_act) {
    const bool last = !c_ok;
    if (!last) {
      if (n_ok && wv == 0) store_rows(st == 2 ? 0 : st + 1, rg);
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
      lds_barrier();                       // X_{p+1}
    }
    p_act = c_act;
    c_si = n_si;
    c_r0 = n_r0;
    c_ok = n_ok;
    st = st == 2 ? 0 : st + 1;
    return !last;
  };
  // The two roles run separate loops under a wave-uniform branch (the
  // kernel is built with the structurizer skipping uniform regions: by
  // default it would sequence the two loops behind flags, and the
  // wait-count insertion would then see one role's loads in flight in the
  // other's loop and stall its matrix work on them).
  if (role == 0) {
    f32x16 s[2];
    bf16x8 wp[2][2];
    for (bool more = c_ok; more;) {  // phases 0 .. n (none without a tile)
      int n_si, n_r0;
      bool n_ok;
      next_tile(n_si, n_r0, n_ok);
      const int ps = st == 0 ? 2 : st - 1;
      const bool c_act = c_ok && pair_active(c_si, c_r0, st);
      if (p_act) mm_tr_p(stage_o(ps), bs.tr, wp, acc);    // dV += dO(T_{p-1})^T P
      if (c_act) mm_rows_p(stage_q(st), bs.row, kv, s);  // S(T_p)
      lds_barrier();                                     // Y_p
      float4 l4[2][4];
      if (c_act) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int m = 0; m < 4; ++m)
            l4[qb][m] = *reinterpret_cast<const float4*>(&s_lse[st][32 * qb + 8 * m + 4 * hf]);
      }
      if (n_ok) issue_loads(n_si, n_r0, st == 2 ? 0 : st + 1, I0{}, I2{});  // two loads of T_{p+1}
      if (c_act) {  // P(T_p): bf16 for dV, fp32 to the dP role through LDS
        const SegArgs g = seg_pick(sg0, sg1, c_si);
        // without document masks, element (qb, m, c) is valid iff
        // 32 qb + 8 m + c >= thr: on a diagonal segment row t sees the key
        // iff t >= key - kv_full, elsewhere every row sees it or none does
        const int thr = g.diag ? key - g.kv_full - c_r0 - 4 * hf : (key < g.kv_full ? -1 : kTileRows);
        // every element valid (wave-uniform): no mask work at all
        const bool dense = !kDoc && __all(thr <= 0);
        auto p_tile = [&](auto masked) {
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
            for (int m = 0; m < 4; ++m) {
              const int rl = 32 * qb + 8 * m + 4 * hf;  // tile row of register 4 m
              const float lv[4] = {l4[qb][m].x, l4[qb][m].y, l4[qb][m].z, l4[qb][m].w};
              int klo[4] = {0, 0, 0, 0}, khi[4] = {a.n_loc, a.n_loc, a.n_loc, a.n_loc};
              if constexpr (kDoc) {
                const int4 lo4 = *reinterpret_cast<const int4*>(&s_klo[st][rl]);
                const int4 hi4 = *reinterpret_cast<const int4*>(&s_khi[st][rl]);
                klo[0] = lo4.x, klo[1] = lo4.y, klo[2] = lo4.z, klo[3] = lo4.w;
                khi[0] = hi4.x, khi[1] = hi4.y, khi[2] = hi4.z, khi[3] = hi4.w;
              }
              float pv[4];
#pragma unroll
              for (int c = 0; c < 4; ++c) {
                const int e = 4 * m + c;
                const float x = __builtin_amdgcn_exp2f(fmaf(s[qb][e], a.scale_log2, -lv[c]));
                if constexpr (decltype(masked)::value) {
                  const int t = c_r0 + rl + c;
                  bool ok;
                  if constexpr (kDoc) ok = key < min(g.kv_full + (g.diag ? t + 1 : 0), khi[c]) && key >= klo[c];
                  else ok = 32 * qb + 8 * m + c >= thr;
                  pv[c] = ok ? x : 0.f;
                } else {
                  pv[c] = x;
                }
                wp[qb][e >> 3][e & 7] = static_cast<__bf16>(pv[c]);
              }
              *reinterpret_cast<float4*>(pbuf + (4 * qb + m) * 256) = make_float4(pv[0], pv[1], pv[2], pv[3]);
            }
          }
        };
        if (dense) p_tile(std::false_type{});
        else p_tile(std::true_type{});
      }
      more = end_phase(n_si, n_r0, n_ok, c_act);
    }
  } else {
    f32x16 dp[2];
    bf16x8 ws[2][2];
    for (bool more = c_ok; more;) {
      int n_si, n_r0;
      bool n_ok;
      next_tile(n_si, n_r0, n_ok);
      const int ps = st == 0 ? 2 : st - 1;
      const bool c_act = c_ok && pair_active(c_si, c_r0, st);
      float4 p4[2][4];
      if (p_act) {  // P of T_{p-1}: these reads first
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int m = 0; m < 4; ++m) p4[qb][m] = *reinterpret_cast<const float4*>(pbuf + (4 * qb + m) * 256);
      }
      if (n_ok) issue_loads(n_si, n_r0, st == 2 ? 0 : st + 1, I2{}, I8{});  // six loads of T_{p+1}
      if (p_act) {  // dS(T_{p-1}) = P (dP - D)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const float4 d4 = *reinterpret_cast<const float4*>(&s_del[ps][32 * qb + 8 * m + 4 * hf]);
            const float dl[4] = {d4.x, d4.y, d4.z, d4.w};
            const float pv[4] = {p4[qb][m].x, p4[qb][m].y, p4[qb][m].z, p4[qb][m].w};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              const int e = 4 * m + c;
              ws[qb][e >> 3][e & 7] = static_cast<__bf16>(pv[c] * (dp[qb][e] - dl[c]));
            }
          }
        }
      }
      lds_barrier();                                      // Y_p
      if (p_act) mm_tr_p(stage_q(ps), bs.tr, ws, acc);    // dK += Q(T_{p-1})^T dS
      if (c_act) mm_rows_p(stage_o(st), bs.row, kv, dp);  // dP(T_p)
      more = end_phase(n_si, n_r0, n_ok, c_act);
    }
  }
  if (!kok) return;
  // lane (key, hf) holds d = 32 b + 8 m + 4 hf + c of its key
  float* dst = (role == 0 ? a.dv : a.dk) + (int64_t(krow) * a.heads + h) * D;
  const float f = role == 0 ? 1.f : a.scale;  // f * x is exactly x for dV
#pragma unroll
  for (int b = 0; b < NB; ++b) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int d0 = 32 * b + 8 * m + 4 * hf;
      float4 x = *reinterpret_cast<float4*>(dst + d0);
      x.x += f * acc[b][4 * m + 0];
      x.y += f * acc[b][4 * m + 1];
      x.z += f * acc[b][4 * m + 2];
      x.w += f * acc[b][4 * m + 3];
      *reinterpret_cast<float4*>(dst + d0) = x;
    }
  }
}

// ---------------------------------------------------------------------------
// Row-major, eight waves: dQ of 256 rows with K/V tiles streamed into LDS.
// ---------------------------------------------------------------------------
// A workgroup of 8 waves owns 256 rows, 32 per wave, whose Q and dO stay in
// registers as the B operand (column = row); per 64-key tile:
//   S^T = K Q^T and dP^T = V dO^T   (A = K / V rows from LDS)
//   P = exp2(S scale log2e - LSE log2e), masked; dS = P (dP - D)
//   dQ^T += K^T dS^T   (A = K read transposed, B = dS^T in register order)
// P is formed in place of S, and the mask is a pass of its own, taken only
// when some row of the wave does not see every key of the tile.  The K/V
// tiles stream through a three-stage direct-to-LDS ring two tiles ahead (a
// tile serves 256 rows): waves 0-3 load the K tile, waves 4-7 the V tile,
// four 1 KiB loads each (tile row 16 (wv & 3) + 4 n + lane / 16, physical
// chunk lane % 16 holding logical chunk (lane % 16) ^ swz(row)).  Keys come
// from the source's two chunks through two buffer bases, so the 32-bit
// offsets stay within one chunk; a tile across the two chunks, or the
// ragged last tile, takes each lane's chunk (at least four loads per wave
// and tile either way).  (Running the two waves of a SIMD half a tile apart,
// as the forward step kernel does, measured slower here: 48 MFMAs per tile
// against little elementwise work leave nothing to overlap.)  A workgroup
// that loaded each tile when it needed it, four waves and 128 rows, took
// 218-220 us per 32k/cp8 rank-0 step against 196-197.
constexpr int kDqRows8 = 256;
constexpr int kDqStages8 = 3;

template <bool kDoc>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads8, kThreads8), amdgpu_waves_per_eu(2, 2)))
void bwd_dq_bf16_d128x8(BwdArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kDqStages8 * 2 * kTileBytes];
  auto kst = [&](int st) { return (lds_u8*)smem + st * 2 * kTileBytes; };
  auto vst = [&](int st) { return (lds_u8*)smem + st * 2 * kTileBytes + kTileBytes; };

  // Dispatch order, longest workgroups first: tile-major over the heads,
  // the segment whose rows see more keys first, and on a diagonal segment
  // its last (longest) rows first.  Each workgroup's result does not depend
  // on the order.
  const int h = blockIdx.x % a.heads;
  int t = blockIdx.x / a.heads;
  auto keys_of = [](const SegArgs& x) { return int64_t(x.kv_full) + (x.diag ? x.q_len : 0); };
  const int s0 = a.nseg == 2 && keys_of(a.seg[1]) > keys_of(a.seg[0]) ? 1 : 0;
  const int si = t < a.seg[s0].tiles ? s0 : 1 - s0;
  if (si != s0) t -= a.seg[s0].tiles;
  const SegArgs g = seg_pick(a.seg[0], a.seg[1], si);
  if (g.diag) t = g.tiles - 1 - t;
  const int row0 = t * kDqRows8;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qc = lane & 31, hf = lane >> 5;
  const int row = row0 + 32 * wv + qc;
  const bool ok = row < g.q_len;
  const int64_t grow = g.q_global + row;
  int prefix = ok ? g.kv_full + (g.diag ? row + 1 : 0) : 0;
  const int w_first = row0 + 32 * wv;
  const int w_last = min(w_first + 32, g.q_len);
  int w_max = w_last > w_first ? g.kv_full + (g.diag ? w_last : 0) : 0;
  int kv_end = g.kv_full + (g.diag ? min(row0 + kDqRows8, g.q_len) : 0);
  // document masks: the row's first key, the wave's smallest first key, the
  // workgroup's first key tile
  int klo = 0, w_lo = 0, kb0 = 0;
  if constexpr (kDoc) {
    int lo, hi;
    doc_row_keys(a, g.q_global + min(row, g.q_len - 1), lo, hi);
    klo = lo;
    prefix = min(prefix, hi);
    doc_row_keys(a, g.q_global + row0, lo, hi);
    kb0 = lo / kTileRows * kTileRows;
    doc_row_keys(a, g.q_global + min(row0 + kDqRows8, g.q_len) - 1, lo, hi);
    kv_end = min(kv_end, hi);
    if (w_last > w_first) {
      doc_row_keys(a, g.q_global + w_first, w_lo, hi);
      doc_row_keys(a, g.q_global + w_last - 1, lo, hi);
      w_max = min(w_max, hi);
    }
  }
  const int ntiles = kv_end > kb0 ? (kv_end - kb0 + kTileRows - 1) / kTileRows : 0;
  const uint32_t row_bytes = uint32_t(a.heads) * 256;
  const uint32_t hoff = uint32_t(h) * 256;

  bf16x8 qf[NT], dof[NT];
  {
    const __bf16* qp = static_cast<const __bf16*>(a.q) + (grow * a.heads + h) * D + 8 * hf;
    const __bf16* dp = static_cast<const __bf16*>(a.dout) + (grow * a.heads + h) * D + 8 * hf;
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      qf[i] = ok ? *reinterpret_cast<const bf16x8*>(qp + 16 * i) : bf16x8{};
      dof[i] = ok ? *reinterpret_cast<const bf16x8*>(dp + 16 * i) : bf16x8{};
    }
  }
  const float lse2 = ok ? a.lse[int64_t(h) * a.seq_len + grow] * kLog2e : INFINITY;
  const float del = ok ? a.delta[int64_t(h) * a.n_loc + g.q_start + row] : 0.f;
  f32x16 dq[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) dq[b] = f32x16{};
  const Bases bs = make_bases(lane);

  // tile loads
  const char* const src = static_cast<const char*>(wv < 4 ? a.k : a.v);
  const dma_u32x4 desc_lo = buffer_desc(src + int64_t(a.kv_lo) * row_bytes, uint32_t(a.kv_split) * row_bytes);
  const dma_u32x4 desc_hi =
      buffer_desc(src + int64_t(a.kv_hi) * row_bytes, uint32_t(max(0, a.kv_valid - a.kv_split)) * row_bytes);
  const int lrow0 = 16 * (wv & 3) + (lane >> 4);  // + 4 n: the lane's tile row for load n
  uint32_t c16[4];                                 // its chunk's byte offset within a row (head included)
#pragma unroll
  for (int n = 0; n < 4; ++n) c16[n] = (uint32_t((lane & 15) ^ swz((lrow0 + 4 * n) & 15)) << 4) + hoff;
  auto issue = [&](int j0, int st) {
    const uint32_t dst = lds_addr((wv < 4 ? kst(st) : vst(st)) + 16 * (wv & 3) * 256);
    const bool whole = j0 + kTileRows <= a.kv_valid && (j0 + kTileRows <= a.kv_split || j0 >= a.kv_split);
    if (whole) {
      const bool lo = j0 < a.kv_split;
      const uint32_t soff = __builtin_amdgcn_readfirstlane(uint32_t(lo ? j0 : j0 - a.kv_split) * row_bytes);
#pragma unroll
      for (int n = 0; n < 4; ++n)
        dma_lds16(lo ? desc_lo : desc_hi, __umul24(uint32_t(lrow0 + 4 * n), row_bytes) + c16[n], soff, dst + n * 1024);
    } else {
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const int kk = min(j0 + lrow0 + 4 * n, a.kv_valid - 1);
        if (kk < a.kv_split)
          dma_lds16(desc_lo, __umul24(uint32_t(kk), row_bytes) + c16[n], 0u, dst + n * 1024);
        else
          dma_lds16(desc_hi, __umul24(uint32_t(kk - a.kv_split), row_bytes) + c16[n], 0u, dst + n * 1024);
      }
    }
  };

  if (ntiles > 0) {
    issue(kb0, 0);
    issue(kb0 + min(1, ntiles - 1) * kTileRows, 1);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the rows above and this wave's first tile loads
  lds_barrier();
  int st = 0;
  for (int j = 0; j < ntiles; ++j) {
    const int j0 = kb0 + j * kTileRows;
    // tile j + 2 into the stage tile j - 1 left (its reads ended before the
    // last barrier)
    issue(kb0 + min(j + 2, ntiles - 1) * kTileRows, st == 0 ? 2 : st - 1);
    if (j0 < w_max && !(kDoc && j0 + kTileRows <= w_lo)) {
      const lds_u8* const tk = kst(st);
      const lds_u8* const tv = vst(st);
      f32x16 s[2], dp[2];
      mm_rows(tk, bs.row, qf, s);
      mm_rows(tv, bs.row, dof, dp);
      // P in place of S; the mask is a pass of its own, taken only when some
      // row of the wave does not see every key of the tile
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) s[kb][e] = __builtin_amdgcn_exp2f(fmaf(s[kb][e], a.scale_log2, -lse2));
      if (kDoc || !__all(!ok || j0 + kTileRows <= prefix)) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int kk = j0 + 32 * kb + 8 * (e >> 2) + 4 * hf + (e & 3);
            if (!(kk < prefix && (!kDoc || kk >= klo))) s[kb][e] = 0.f;
          }
      }
      bf16x8 ws[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) ws[kb][e >> 3][e & 7] = static_cast<__bf16>(s[kb][e] * (dp[kb][e] - del));
      mm_tr(tk, bs.tr, ws, dq);
    }
    // tile j + 1 has landed (loads complete in order; at least four loads,
    // those of tile j + 2, were issued since)
    __builtin_amdgcn_s_waitcnt(0x0F74);  // vmcnt(4)
    lds_barrier();
    st = st == 2 ? 0 : st + 1;
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): no load in flight at exit
  if (!ok) return;
  float* dqp = a.dq + (grow * a.heads + h) * D;
  const bool first = g.epi != 0;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int d0 = 32 * b + 8 * m + 4 * hf;
      float4 x = first ? make_float4(0.f, 0.f, 0.f, 0.f) : *reinterpret_cast<float4*>(dqp + d0);
      x.x += a.scale * dq[b][4 * m + 0];
      x.y += a.scale * dq[b][4 * m + 1];
      x.z += a.scale * dq[b][4 * m + 2];
      x.w += a.scale * dq[b][4 * m + 3];
      *reinterpret_cast<float4*>(dqp + d0) = x;
    }
  }
}

}  // namespace

bool bwd_mfma(int dtype_bf16, int head_dim) { return dtype_bf16 && head_dim == 128; }
int bwd_mfma_rows() { return kDqRows8; }
int bwd_mfma_keys() { return kKeys; }

template <bool kDoc>
hipError_t launch_bf16_d128(const BwdArgs& a, bool eight, hipStream_t st) {
  if (a.key_tiles > 0) {
    const unsigned grid = unsigned(a.key_tiles) * unsigned(a.heads);
    if (eight) bwd_dkdv_bf16_d128x8<kDoc><<<grid, kThreads8, 0, st>>>(a);
    else bwd_dkdv_bf16_d128<kDoc><<<grid, kThreads, 0, st>>>(a);
  }
  if (a.total_tiles > 0) bwd_dq_bf16_d128x8<kDoc><<<unsigned(a.total_tiles) * unsigned(a.heads), kThreads8, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_bwd_bf16_d128(const BwdArgs& a, bool eight_wave_keys, hipStream_t st) {
  return a.doc ? launch_bf16_d128<true>(a, eight_wave_keys, st) : launch_bf16_d128<false>(a, eight_wave_keys, st);
}

}  // namespace cpattn
