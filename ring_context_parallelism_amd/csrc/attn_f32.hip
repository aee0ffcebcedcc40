// fp32 blockwise step attention (one ring step of one rank), gfx950.
//
// The plain-precision path for fp32 inputs: every product and sum in fp32 on
// the vector ALUs, no reduced-precision operand anywhere.  A workgroup owns 64
// query rows of one head; four lanes share a row, each holding a quarter of
// the head dimension.  K/V tiles of 32 keys are staged in LDS and the row's
// softmax is updated online (running max m, running sum l, rescaled O), the
// blockwise K/V update of "Sequence Parallelism IV: Megatron Context Parallel
// and Load-Balanced Rings", section 4 "What Actually Moves".  Each row sees a
// prefix of the source's local K/V buffer given by its segment (kv_full keys,
// plus keys up to its own position on a diagonal chunk); tiles past the
// workgroup's longest prefix are never loaded -- the skipped future
// sub-blocks of the same section.
#include <hip/hip_runtime.h>

#include <cmath>

#include "epilogue.h"
#include "kernels.h"

namespace cpattn {
namespace {

constexpr int kBM = 64;   // rows per workgroup
constexpr int kBN = 32;   // keys per LDS tile
constexpr int kTPR = 4;   // lanes per row
constexpr int kThreads = kBM * kTPR;

template <int D>
__global__ __launch_bounds__(kThreads) void attn_step_f32(StepArgs a) {
  constexpr int DS = D / kTPR;  // head-dim values per lane
  constexpr int LS = D + 4;     // LDS row stride (floats)
  __shared__ float sk[kBN * LS];
  __shared__ float sv[kBN * LS];

  const int h = blockIdx.x / a.total_tiles;
  int t = blockIdx.x % a.total_tiles;
  const int si = t < a.seg[0].tiles ? 0 : 1;
  if (si) t -= a.seg[0].tiles;
  const SegArgs& g = a.seg[si];
  const int epi = __builtin_amdgcn_readfirstlane(g.epi);  // scalar: the epilogue branches on it
  const int row0 = t * kBM;
  const int tid = threadIdx.x;
  const int rl = tid / kTPR, sub = tid % kTPR;
  const int row = row0 + rl;  // row within the segment
  const bool ok = row < g.q_len;
  int prefix = ok ? g.kv_full + (g.diag ? row + 1 : 0) : 0;
  const int last = min(row0 + kBM, g.q_len);
  int kv_end = g.kv_full + (g.diag ? last : 0);
  // document masks: a row sees only its document's run of the source's keys,
  // [klo, khi); the rows are consecutive positions, so the workgroup's keys
  // run from its first row's klo to its last row's khi
  int klo = 0, kb0 = 0;
  if (a.doc) {
    int lo, hi;
    doc_row_keys(a, g.q_global + min(row, g.q_len - 1), lo, hi);
    klo = lo;
    prefix = min(prefix, hi);
    doc_row_keys(a, g.q_global + row0, lo, hi);
    kb0 = lo / kBN * kBN;
    doc_row_keys(a, g.q_global + last - 1, lo, hi);
    kv_end = min(kv_end, hi);
  }

  const float* q = static_cast<const float*>(a.q);
  const float* kp = static_cast<const float*>(a.k);
  const float* vp = static_cast<const float*>(a.v);
  const int64_t grow = g.q_global + row;

  float qv[DS];
  float o[DS];
#pragma unroll
  for (int i = 0; i < DS; ++i) {
    qv[i] = ok ? q[(grow * a.heads + h) * D + sub * DS + i] : 0.f;
    o[i] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  if (a.tile_cnt && tid == 0)  // work counter: the workgroup computes every key tile from kb0 below kv_end
    __hip_atomic_fetch_add(a.tile_cnt, (unsigned long long)max(0, (kv_end + kBN - 1) / kBN - kb0 / kBN),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  for (int j0 = kb0; j0 < kv_end; j0 += kBN) {
    __syncthreads();
    for (int e = tid; e < kBN * D; e += kThreads) {
      const int kr = e / D, dc = e % D;
      const int key = j0 + kr;
      float kx = 0.f, vx = 0.f;
      if (key < a.kv_valid) {  // keys past the real ones stay zero (and masked)
        const int64_t off = (int64_t(kv_row(a, key)) * a.heads + h) * D + dc;
        kx = kp[off];
        vx = vp[off];
      }
      sk[kr * LS + dc] = kx;
      sv[kr * LS + dc] = vx;
    }
    __syncthreads();

    float sc[kBN];
    float mt = -INFINITY;
#pragma unroll
    for (int kk = 0; kk < kBN; ++kk) {
      float part = 0.f;
#pragma unroll
      for (int i = 0; i < DS; ++i) part = fmaf(qv[i], sk[kk * LS + sub * DS + i], part);
      part += __shfl_xor(part, 1);
      part += __shfl_xor(part, 2);
      sc[kk] = (j0 + kk < prefix && j0 + kk >= klo) ? part * a.scale : -INFINITY;
      mt = fmaxf(mt, sc[kk]);
    }
    const float mn = fmaxf(m, mt);
    const float alpha = (m == -INFINITY) ? 0.f : expf(m - mn);
    l *= alpha;
#pragma unroll
    for (int i = 0; i < DS; ++i) o[i] *= alpha;
#pragma unroll
    for (int kk = 0; kk < kBN; ++kk) {
      const float p = (sc[kk] == -INFINITY) ? 0.f : expf(sc[kk] - mn);
      l += p;
#pragma unroll
      for (int i = 0; i < DS; ++i) o[i] = fmaf(p, sv[kk * LS + sub * DS + i], o[i]);
    }
    m = mn;
  }

  if (!ok) return;
  const int lrow = g.q_start + row;
  const float lse_s = m + logf(l);
  const float inv = l > 0.f ? 1.f / l : 0.f;  // a row that saw no key (document masks): O_s = 0, lse_s = -inf
  if (a.doc && l == 0.f && epi == kEpiMerge) return;  // ... and leaves a merge-only step's running state as it is
  float4 c[DS / 4];
#pragma unroll
  for (int i = 0; i < DS; i += 4) c[i / 4] = row_epi_load4(a, epi, h, lrow, sub * DS + i, D);
  const RowEpi e = row_epi_begin(a, epi, h, lrow, lse_s);
#pragma unroll
  for (int i = 0; i < DS; i += 4) {
    float4 v4 = make_float4(o[i] * inv, o[i + 1] * inv, o[i + 2] * inv, o[i + 3] * inv);
    row_epi_store4(a, epi, e, h, lrow, grow, sub * DS + i, D, v4, c[i / 4]);
  }
  if (sub == 0) row_epi_store_lse(a, epi, e, h, lrow, grow, lse_s);
}

}  // namespace

int attn_f32_block_m() { return kBM; }
int attn_f32_block_n() { return kBN; }

hipError_t launch_attn_f32(const StepArgs& a, int head_dim, hipStream_t stream) {
  const dim3 grid(unsigned(a.total_tiles) * unsigned(a.heads));
  if (head_dim == 128) {
    attn_step_f32<128><<<grid, kThreads, 0, stream>>>(a);
  } else {
    attn_step_f32<64><<<grid, kThreads, 0, stream>>>(a);
  }
  return hipGetLastError();
}

}  // namespace cpattn
