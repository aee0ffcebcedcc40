// Step epilogue shared by the attention kernels: turn one row's step result
// (normalised O_s, lse_s) into the running state, a partial, or the output.
//
// Exact merge ("Sequence Parallelism IV: Megatron Context Parallel and
// Load-Balanced Rings", section 4 "What Actually Moves": carrying the running
// max and sum from block to block makes the split computation equal the
// unsplit softmax).  In (O, LSE) form:
//   lse' = max(a, b) + log1p(exp(-|a - b|)),
//   O'   = exp(a - lse') O_acc + exp(b - lse') O_s,
// where a = lse_acc, b = lse_s; an empty state (a = -inf) takes the partial.
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>

#include "kernels.h"

namespace cpattn {

// Source row of local key kk (0 <= kk < kv_valid) in the step's K/V tensors.
__device__ __forceinline__ int kv_row(const StepArgs& a, int kk) {
  return kk < a.kv_split ? a.kv_lo + kk : a.kv_hi + (kk - a.kv_split);
}

// Document masks: local keys of the step's source below global position x
// (the source's local keys are in increasing position order).  A is StepArgs
// or BwdArgs.
template <typename A>
__device__ __forceinline__ int doc_keys_before(const A& a, int x) {
  return min(max(x - a.kpos_lo, 0), a.kpos_split) + min(max(x - a.kpos_hi, 0), a.n_loc - a.kpos_split);
}

// The run of local keys [lo, hi) of the document holding global position grow.
template <typename A>
__device__ __forceinline__ void doc_row_keys(const A& a, int64_t grow, int& lo, int& hi) {
  const int2 d = reinterpret_cast<const int2*>(a.doc)[grow];
  lo = doc_keys_before(a, d.x);
  hi = doc_keys_before(a, d.y);
}

struct RowEpi {
  float wa;  // weight of the running state (0: not read)
  float ws;  // weight of this step's partial
  float L;   // resulting LSE (natural log)
};

// epi is the segment's EpiMode flags, wave-uniform (pass it through
// readfirstlane so the mode tests are scalar branches).
__device__ __forceinline__ RowEpi row_epi_begin(const StepArgs& a, int epi, int h, int lrow, float lse_s) {
  RowEpi e{0.f, 1.f, lse_s};
  if ((epi & 3) == kEpiMerge) {
    const float la = a.acc_lse[int64_t(h) * a.n_loc + lrow];
    if (la != -INFINITY) {
      if (lse_s == -INFINITY) {
        e.wa = 1.f;
        e.ws = 0.f;
        e.L = la;
      } else {
        const float mx = fmaxf(la, lse_s);
        const float L = mx + log1pf(expf(-fabsf(la - lse_s)));
        e.wa = expf(la - L);
        e.ws = expf(lse_s - L);
        e.L = L;
      }
    }
  }
  return e;
}

// Running-state O values d0..d0+3 of local row lrow, head h, that a merge
// reads (zero otherwise).  A row's loads are all issued before its stores
// (and without waiting for row_epi_begin's LSE read: the values are only used
// where that weight is nonzero), so they are in flight together instead of
// one memory round trip per four values.
__device__ __forceinline__ float4 row_epi_load4(const StepArgs& a, int epi, int h, int lrow, int d0, int head_dim) {
  if ((epi & 3) != kEpiMerge) return make_float4(0.f, 0.f, 0.f, 0.f);
  return *reinterpret_cast<const float4*>(a.acc_o + (int64_t(lrow) * a.heads + h) * head_dim + d0);
}

// Four consecutive head-dim values d0..d0+3 of local row lrow, head h: o is
// this step's normalised output, c what row_epi_load4 returned for them.
__device__ __forceinline__ void row_epi_store4(const StepArgs& a, int epi, const RowEpi& e, int h, int lrow,
                                               int64_t grow, int d0, int head_dim, float4 o, float4 c) {
  const int mode = epi & 3;
  const int64_t lidx = (int64_t(lrow) * a.heads + h) * head_dim + d0;
  if (mode == kEpiPartial) {
    *reinterpret_cast<float4*>(a.part_o + lidx) = o;
    return;
  }
  float4 r = make_float4(o.x * e.ws, o.y * e.ws, o.z * e.ws, o.w * e.ws);
  if (e.wa != 0.f) {  // an empty running state (weight 0) may hold anything, even NaN
    r.x += e.wa * c.x;
    r.y += e.wa * c.y;
    r.z += e.wa * c.z;
    r.w += e.wa * c.w;
  }
  if (epi & kEpiFinal) {
    const int64_t gidx = (grow * a.heads + h) * head_dim + d0;
    if (a.out_f32) {
      *reinterpret_cast<float4*>(static_cast<float*>(a.out) + gidx) = r;
    } else {
      __bf16* op = static_cast<__bf16*>(a.out) + gidx;
      typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
      bf16x4 b;
      b[0] = static_cast<__bf16>(r.x);
      b[1] = static_cast<__bf16>(r.y);
      b[2] = static_cast<__bf16>(r.z);
      b[3] = static_cast<__bf16>(r.w);
      *reinterpret_cast<bf16x4*>(op) = b;
    }
  } else {
    *reinterpret_cast<float4*>(a.acc_o + lidx) = r;
  }
}

__device__ __forceinline__ void row_epi_store_lse(const StepArgs& a, int epi, const RowEpi& e, int h, int lrow,
                                                  int64_t grow, float lse_s) {
  const int mode = epi & 3;
  if (mode == kEpiPartial) {
    a.part_lse[int64_t(h) * a.n_loc + lrow] = lse_s;
  } else if (epi & kEpiFinal) {
    a.lse[int64_t(h) * a.seq_len + grow] = e.L;
  } else {
    a.acc_lse[int64_t(h) * a.n_loc + lrow] = e.L;
  }
}

}  // namespace cpattn
