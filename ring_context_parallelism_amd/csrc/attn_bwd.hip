// Backward of one ring step of one rank (gfx950): the gradients of the rank's
// queries and of the source's keys and values over the step's valid pairs.
//
// "Context Parallelism for Long-Context Training", section "Prove attention
// equivalence", asks for gradients equal to the unsharded reference.  With the
// complete forward's LSE and O, the softmax of a valid pair is known exactly
// in every step, P_ij = exp(s_ij - LSE_i), so the steps need no merge: each
// adds its pairs' terms
//   dV_j += P_ij dO_i,  dS_ij = P_ij (<dO_i, v_j> - D_i),  D_i = <dO_i, O_i>,
//   dQ_i += scale dS_ij k_j,  dK_j += scale dS_ij q_i
// to the rank's dQ and to the source's dK, dV.  The valid pairs of a step are
// the forward's ("Sequence Parallelism IV: Megatron Context Parallel and
// Load-Balanced Rings", section 4): each local row sees a prefix of the
// source's local K/V buffer; sub-blocks past it are skipped.
//
// Two kernels per step, so that no gradient needs atomics:
//   * key-major: a workgroup owns a tile of the source's keys and walks the
//     rank's rows that see them, accumulating dK and dV in registers; it is
//     the only writer of those key rows in the launch (read-modify-write of
//     the fp32 gradient, which collects every rank's terms);
//   * row-major: a workgroup owns a tile of the rank's rows and walks the
//     keys they see, accumulating dQ (written at the row run's first step,
//     added to afterwards).
// Document masks clip every row's keys to its document's run of the source,
// [klo, khi) (rows of a segment are consecutive positions, so both grow with
// the row).  Plus a per-rank kernel for D_i.  This file holds the generic kernels (any
// element type, fp32 arithmetic on the vector ALUs); the bf16 head_dim 128
// kernels on the matrix cores are in attn_bwd_bf16.hip.
#include <hip/hip_runtime.h>

#include <cmath>

#include "epilogue.h"
#include "kernels.h"

namespace cpattn {
namespace {

constexpr int kThreads = 256;
constexpr int kSub = 8;   // lanes sharing a key (key-major) or a row (row-major)
constexpr int kTile = 32; // keys per key-major workgroup, rows per row-major workgroup; LDS tile rows
constexpr float kLog2e = 1.4426950408889634f;

template <typename T>
__device__ __forceinline__ float ld(const T* p) {
  return static_cast<float>(*p);
}

__device__ __forceinline__ float sum_sub(float x) {  // over the kSub lanes of a group
  x += __shfl_xor(x, 1);
  x += __shfl_xor(x, 2);
  x += __shfl_xor(x, 4);
  return x;
}

// D_i = <dO_i, O_i> of the rank's real local rows.  One item = (head, row):
// D / kVec lanes per item, each with one 16-byte vector of O and of dO, then
// a shuffle reduction within the item's lanes (an aligned power-of-two group
// of a wave).
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void bwd_delta(BwdArgs a) {
  constexpr int kVec = 16 / int(sizeof(T));  // elements per 16-byte vector
  constexpr int kLanes = D / kVec;           // lanes per item: 8 to 32
  static_assert(kLanes >= 1 && kLanes <= 64 && (kLanes & (kLanes - 1)) == 0, "lanes per item");
  const int64_t gtid = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  const int64_t item = gtid / kLanes;
  const int sub = int(gtid % kLanes);
  const int64_t rows = a.delta_rows;
  const bool ok = item < rows * a.heads;  // lanes past the end still join the shuffles
  const int h = ok ? int(item / rows) : 0;
  const int lrow = ok ? int(item % rows) : 0;
  float s = 0.f;
  if (ok) {
    const int64_t grow = lrow < a.delta_split ? a.delta_lo + lrow : a.delta_hi + (lrow - a.delta_split);
    const int64_t off = (grow * a.heads + h) * D + sub * kVec;
    typedef T tv __attribute__((ext_vector_type(kVec)));
    const tv o = *reinterpret_cast<const tv*>(static_cast<const T*>(a.out) + off);
    const tv d = *reinterpret_cast<const tv*>(static_cast<const T*>(a.dout) + off);
#pragma unroll
    for (int i = 0; i < kVec; ++i) s = fmaf(static_cast<float>(o[i]), static_cast<float>(d[i]), s);
  }
#pragma unroll
  for (int m = kLanes / 2; m >= 1; m >>= 1) s += __shfl_xor(s, m);
  if (ok && sub == 0) a.delta[int64_t(h) * a.n_loc + lrow] = s;
}

__device__ __forceinline__ int bwd_kv_row(const BwdArgs& a, int kk) {
  return kk < a.kv_split ? a.kv_lo + kk : a.kv_hi + (kk - a.kv_split);
}

// Key-major: kTile keys of one head, kSub lanes per key (dims sub, sub + kSub, ...).
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void bwd_dkdv_generic(BwdArgs a) {
  constexpr int DS = D / kSub;
  __shared__ float sq[kTile * D];
  __shared__ float sdo[kTile * D];
  __shared__ float slse[kTile];
  __shared__ float sdel[kTile];
  __shared__ int sklo[kTile];  // document masks: the rows' key runs
  __shared__ int skhi[kTile];

  const int h = blockIdx.x % a.heads;
  const int k0 = (blockIdx.x / a.heads) * kTile;
  const int tid = threadIdx.x;
  const int kl = tid / kSub, sub = tid % kSub;
  const int key = k0 + kl;
  const bool kok = key < a.kv_valid;

  const T* kp = static_cast<const T*>(a.k);
  const T* vp = static_cast<const T*>(a.v);
  float kv[DS], vv[DS], dk[DS], dv[DS];
  const int64_t krow = kok ? bwd_kv_row(a, key) : 0;
#pragma unroll
  for (int i = 0; i < DS; ++i) {
    kv[i] = kok ? ld(kp + (krow * a.heads + h) * D + i * kSub + sub) : 0.f;
    vv[i] = kok ? ld(vp + (krow * a.heads + h) * D + i * kSub + sub) : 0.f;
    dk[i] = 0.f;
    dv[i] = 0.f;
  }
  const T* qp = static_cast<const T*>(a.q);
  const T* dop = static_cast<const T*>(a.dout);

  for (int si = 0; si < a.nseg; ++si) {
    const SegArgs& g = a.seg[si];
    // rows that see a key of this tile: all if the tile starts inside the
    // segment's full prefix, else (diagonal) from the first row whose own
    // prefix reaches the tile
    int t0;
    if (k0 < g.kv_full) t0 = 0;
    else if (g.diag) t0 = k0 - g.kv_full;  // row t sees keys < kv_full + t + 1
    else continue;
    for (int r0 = t0; r0 < g.q_len; r0 += kTile) {
      __syncthreads();
      for (int e = tid; e < kTile * D; e += kThreads) {
        const int rr = e / D, c = e % D;
        const int t = r0 + rr;
        float x = 0.f, y = 0.f;
        if (t < g.q_len) {
          const int64_t grow = g.q_global + t;
          x = ld(qp + (grow * a.heads + h) * D + c);
          y = ld(dop + (grow * a.heads + h) * D + c);
        }
        sq[e] = x;
        sdo[e] = y;
      }
      if (tid < kTile) {
        const int t = r0 + tid;
        const bool ok = t < g.q_len;
        slse[tid] = ok ? a.lse[int64_t(h) * a.seq_len + g.q_global + t] * kLog2e : 0.f;
        sdel[tid] = ok ? a.delta[int64_t(h) * a.n_loc + g.q_start + t] : 0.f;
        int lo = 0, hi = a.n_loc;
        if (a.doc && ok) doc_row_keys(a, g.q_global + t, lo, hi);
        sklo[tid] = lo;
        skhi[tid] = hi;
      }
      __syncthreads();
      const int rn = min(kTile, g.q_len - r0);
      for (int rr = 0; rr < rn; ++rr) {
        const int t = r0 + rr;
        float s = 0.f, dp = 0.f;
#pragma unroll
        for (int i = 0; i < DS; ++i) {
          s = fmaf(sq[rr * D + i * kSub + sub], kv[i], s);
          dp = fmaf(sdo[rr * D + i * kSub + sub], vv[i], dp);
        }
        s = sum_sub(s);
        dp = sum_sub(dp);
        const bool valid = kok && key < g.kv_full + (g.diag ? t + 1 : 0) && key >= sklo[rr] && key < skhi[rr];
        const float p = valid ? exp2f(s * a.scale_log2 - slse[rr]) : 0.f;
        const float ds = p * (dp - sdel[rr]);
#pragma unroll
        for (int i = 0; i < DS; ++i) {
          dv[i] = fmaf(p, sdo[rr * D + i * kSub + sub], dv[i]);
          dk[i] = fmaf(ds, sq[rr * D + i * kSub + sub], dk[i]);
        }
      }
    }
  }
  if (!kok) return;
  float* dkp = a.dk + (krow * a.heads + h) * D;
  float* dvp = a.dv + (krow * a.heads + h) * D;
#pragma unroll
  for (int i = 0; i < DS; ++i) {
    dkp[i * kSub + sub] += a.scale * dk[i];
    dvp[i * kSub + sub] += dv[i];
  }
}

// Row-major: kTile rows of one segment and head, kSub lanes per row.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void bwd_dq_generic(BwdArgs a) {
  constexpr int DS = D / kSub;
  __shared__ float sk[kTile * D];
  __shared__ float sv[kTile * D];

  const int h = blockIdx.x / a.total_tiles;
  int t = blockIdx.x % a.total_tiles;
  const int si = t < a.seg[0].tiles ? 0 : 1;
  if (si) t -= a.seg[0].tiles;
  const SegArgs& g = a.seg[si];
  const int row0 = t * kTile;
  const int tid = threadIdx.x;
  const int rl = tid / kSub, sub = tid % kSub;
  const int row = row0 + rl;
  const bool ok = row < g.q_len;
  int prefix = ok ? g.kv_full + (g.diag ? row + 1 : 0) : 0;
  int kv_end = g.kv_full + (g.diag ? min(row0 + kTile, g.q_len) : 0);
  const int64_t grow = g.q_global + row;
  int klo = 0, kb0 = 0;  // document masks: the row's first key, the workgroup's first key tile
  if (a.doc) {
    int lo, hi;
    doc_row_keys(a, g.q_global + min(row, g.q_len - 1), lo, hi);
    klo = lo;
    prefix = min(prefix, hi);
    doc_row_keys(a, g.q_global + row0, lo, hi);
    kb0 = lo / kTile * kTile;
    doc_row_keys(a, g.q_global + min(row0 + kTile, g.q_len) - 1, lo, hi);
    kv_end = min(kv_end, hi);
  }

  const T* qp = static_cast<const T*>(a.q);
  const T* dop = static_cast<const T*>(a.dout);
  float qv[DS], dov[DS], dq[DS];
#pragma unroll
  for (int i = 0; i < DS; ++i) {
    qv[i] = ok ? ld(qp + (grow * a.heads + h) * D + i * kSub + sub) : 0.f;
    dov[i] = ok ? ld(dop + (grow * a.heads + h) * D + i * kSub + sub) : 0.f;
    dq[i] = 0.f;
  }
  const float lse2 = ok ? a.lse[int64_t(h) * a.seq_len + grow] * kLog2e : 0.f;
  const float del = ok ? a.delta[int64_t(h) * a.n_loc + g.q_start + row] : 0.f;

  const T* kp = static_cast<const T*>(a.k);
  const T* vp = static_cast<const T*>(a.v);
  for (int j0 = kb0; j0 < kv_end; j0 += kTile) {
    __syncthreads();
    for (int e = tid; e < kTile * D; e += kThreads) {
      const int kr = e / D, c = e % D;
      const int key = j0 + kr;
      float x = 0.f, y = 0.f;
      if (key < a.kv_valid) {
        const int64_t off = (int64_t(bwd_kv_row(a, key)) * a.heads + h) * D + c;
        x = ld(kp + off);
        y = ld(vp + off);
      }
      sk[e] = x;
      sv[e] = y;
    }
    __syncthreads();
    const int jn = min(kTile, kv_end - j0);
    for (int kk = 0; kk < jn; ++kk) {
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int i = 0; i < DS; ++i) {
        s = fmaf(qv[i], sk[kk * D + i * kSub + sub], s);
        dp = fmaf(dov[i], sv[kk * D + i * kSub + sub], dp);
      }
      s = sum_sub(s);
      dp = sum_sub(dp);
      const float p = (j0 + kk < prefix && j0 + kk >= klo) ? exp2f(s * a.scale_log2 - lse2) : 0.f;
      const float ds = p * (dp - del);
#pragma unroll
      for (int i = 0; i < DS; ++i) dq[i] = fmaf(ds, sk[kk * D + i * kSub + sub], dq[i]);
    }
  }
  if (!ok) return;
  float* dqp = a.dq + (grow * a.heads + h) * D;
  const bool first = g.epi != 0;
#pragma unroll
  for (int i = 0; i < DS; ++i) {
    const float x = a.scale * dq[i];
    dqp[i * kSub + sub] = first ? x : dqp[i * kSub + sub] + x;
  }
}

template <typename T, int D>
hipError_t launch_generic(const BwdArgs& a, hipStream_t st) {
  if (a.key_tiles > 0) bwd_dkdv_generic<T, D><<<unsigned(a.key_tiles) * unsigned(a.heads), kThreads, 0, st>>>(a);
  if (a.total_tiles > 0) bwd_dq_generic<T, D><<<unsigned(a.total_tiles) * unsigned(a.heads), kThreads, 0, st>>>(a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_delta_t(const BwdArgs& a, hipStream_t st) {
  const int64_t items = a.delta_rows * a.heads;
  if (items == 0) return hipSuccess;
  const int64_t threads = items * (D / (16 / int64_t(sizeof(T))));
  bwd_delta<T, D><<<unsigned((threads + kThreads - 1) / kThreads), kThreads, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace

int bwd_generic_tile() { return kTile; }

hipError_t launch_bwd_delta(const BwdArgs& a, int dtype_bf16, int head_dim, hipStream_t st) {
  if (dtype_bf16) return head_dim == 128 ? launch_delta_t<__bf16, 128>(a, st) : launch_delta_t<__bf16, 64>(a, st);
  return head_dim == 128 ? launch_delta_t<float, 128>(a, st) : launch_delta_t<float, 64>(a, st);
}

hipError_t launch_bwd_generic(const BwdArgs& a, int dtype_bf16, int head_dim, hipStream_t st) {
  if (dtype_bf16) return head_dim == 128 ? launch_generic<__bf16, 128>(a, st) : launch_generic<__bf16, 64>(a, st);
  return head_dim == 128 ? launch_generic<float, 128>(a, st) : launch_generic<float, 64>(a, st);
}

}  // namespace cpattn
