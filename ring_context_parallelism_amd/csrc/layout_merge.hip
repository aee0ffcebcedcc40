// Bandwidth-bound kernels: zigzag/contiguous layout copies (also the one-GPU
// ring receive), NaN poisoning, the separate LSE merge, and finalize.
//
// Layout ("Sequence Parallelism IV: Megatron Context Parallel and
// Load-Balanced Rings", section 3): rank r's local rows are chunk r followed
// by chunk 2cp-1-r (zigzag), or the contiguous slice r.  Each token row is
// heads*head_dim elements and is moved as whole 16-byte vectors; one
// workgroup walks whole rows so the row -> global-token arithmetic is done
// once per row.
//
// Merge (section 4 "What Actually Moves"): the running state and a step's
// partial are folded with log-sum-exp weights, which is exact.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "kernels.h"

namespace cpattn {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ int64_t local_to_global(int64_t r, int64_t li, int64_t chunk, int64_t n_loc, int cp,
                                                   int zigzag) {
  if (!zigzag) return r * n_loc + li;
  const bool late = li >= chunk;
  const int64_t ch = late ? 2 * int64_t(cp) - 1 - r : r;
  return ch * chunk + (late ? li - chunk : li);
}

// One workgroup per row (grid-stride over rows): the row -> token arithmetic
// is done once per row, then the row's 16-byte vectors are copied.
__global__ __launch_bounds__(kThreads) void layout_copy(LayoutArgs a) {
  const int tsel = blockIdx.y;
  const uint4* src = static_cast<const uint4*>(a.src[tsel]);
  uint4* dst = static_cast<uint4*>(a.dst[tsel]);
  const int64_t rows = int64_t(a.rank_count) * a.n_loc;
  for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
    const int64_t r = a.rank_begin + row / a.n_loc;
    const int64_t li = row % a.n_loc;
    const int64_t g = local_to_global(r, li, a.chunk, a.n_loc, a.cp, a.zigzag);
    const int64_t lrow = (r - a.dst_rank0) * a.n_loc + li;
    if (g >= a.seq_len) {  // pad row: zero in the local layout, absent from the natural one
      if (a.to_local)
        for (int64_t c = threadIdx.x; c < a.row_vec; c += kThreads) dst[lrow * a.row_vec + c] = uint4{0u, 0u, 0u, 0u};
      continue;
    }
    const int64_t from = (a.to_local ? g : lrow) * a.row_vec;
    const int64_t to = (a.to_local ? lrow : g) * a.row_vec;
    for (int64_t c = threadIdx.x; c < a.row_vec; c += kThreads) dst[to + c] = src[from + c];
  }
}

// Ulysses all-to-all ("Sequence Parallelism IV: Megatron Context Parallel and
// Load-Balanced Rings", section 7 "CP vs Ulysses": ranks trade their token
// slices so that each ends up with all tokens of a subset of heads).  A (head owner r', token t) row of
// the head layout -- the H/cp heads of token t that r' receives -- is one
// contiguous run of `run` 16-byte vectors in the sequence owner's local row,
// so both sides move whole vectors.  Each thread moves one vector of a row
// (a workgroup covers kThreads / run rows when a run is shorter than the
// workgroup); the row arithmetic is 32-bit (the plan keeps every tensor below
// 2^32 bytes, so rows and vector indices fit).
__global__ __launch_bounds__(kThreads) void ulysses_copy(UlyssesArgs a) {
  const uint4* src = static_cast<const uint4*>(a.src);
  uint4* dst = static_cast<uint4*>(a.dst);
  const uint32_t group = uint32_t(a.heads / a.cp);
  const uint32_t run = group * uint32_t(a.head_vec);     // vectors per (r', t)
  const uint32_t tpr = run < uint32_t(kThreads) ? run : uint32_t(kThreads);  // threads per row
  const uint32_t rpw = uint32_t(kThreads) / tpr;          // rows per workgroup pass
  const uint32_t sub = threadIdx.x / tpr, lv = threadIdx.x % tpr;
  if (sub >= rpw) return;
  const uint32_t seq = uint32_t(a.seq_len), chunk = uint32_t(a.chunk), cp = uint32_t(a.cp);
  const uint32_t rows = cp * seq;
  for (uint32_t row = blockIdx.x * rpw + sub; row < rows; row += gridDim.x * rpw) {
    const uint32_t rh = row / seq, t = row - rh * seq;
    const uint32_t c = t / chunk, tc = t - c * chunk;
    uint32_t owner, li;
    if (a.zigzag) {
      owner = c < cp ? c : 2 * cp - 1 - c;
      li = (c < cp ? 0 : chunk) + tc;
    } else {
      owner = c;
      li = tc;
    }
    const uint32_t hs = row * run;                                                                  // head layout
    const uint32_t sq = ((owner * uint32_t(a.n_loc) + li) * uint32_t(a.heads) + rh * group) * uint32_t(a.head_vec);
    const uint32_t from = a.to_heads ? sq : hs;
    const uint32_t to = a.to_heads ? hs : sq;
    for (uint32_t v = lv; v < run; v += tpr) dst[to + v] = src[from + v];
  }
}

// Ring receive as a kernel of its own on the copy stream: one wave per
// workgroup and at most 16 VGPRs, so its waves fit in the registers the step
// kernel leaves free on each SIMD and the copy runs beside the step instead
// of taking compute units from it (and with its own memory counters, so the
// step never waits for the copy's stores).  Each lane keeps two non-temporal
// 16-byte loads in flight; offsets are 32-bit from scalar bases (a range is
// below 4 GiB: the plan bounds every tensor to 2^32 bytes).
__global__ __launch_bounds__(64) __attribute__((amdgpu_num_vgpr(16))) void recv_copy(RecvArgs a) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(1))) u32x4 g_u32x4;
  typedef __attribute__((address_space(1))) const char g_cchar;
  typedef __attribute__((address_space(1))) char g_char;
  const uint32_t stride = gridDim.x * 64u * 16u;  // bytes
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if (r >= a.n) break;
    g_cchar* src = (g_cchar*)(a.src[r]);
    g_char* dst = (g_char*)(a.dst[r]);
    const uint32_t n = uint32_t(a.vec[r]) * 16u;
    uint32_t o = (blockIdx.x * 64u + threadIdx.x) * 16u;
    for (; o + stride < n; o += 2 * stride) {
      const uint32_t o1 = o + stride;
      const u32x4 x0 = __builtin_nontemporal_load((const g_u32x4*)(src + o));
      const u32x4 x1 = __builtin_nontemporal_load((const g_u32x4*)(src + o1));
      __builtin_nontemporal_store(x0, (g_u32x4*)(dst + o));
      __builtin_nontemporal_store(x1, (g_u32x4*)(dst + o1));
    }
    if (o < n) __builtin_nontemporal_store(__builtin_nontemporal_load((const g_u32x4*)(src + o)), (g_u32x4*)(dst + o));
  }
}

// Fused-ring receive flag: launched behind the copy kernel on its stream, so
// it runs once that kernel has completed (and its writes are visible at agent
// scope); the release store then publishes the call's epoch, which a kernel
// on the caller's stream advanced before the copy stream started (so a
// replayed graph publishes a new one each time).
__global__ __launch_bounds__(64) void ring_signal(uint32_t* flag, const uint32_t* epoch) {
  if (threadIdx.x == 0) __hip_atomic_store(flag, *epoch, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

// The same with the epoch passed by value (calls not recorded into a graph:
// the host numbers them, and no kernel has to advance a device word first).
__global__ __launch_bounds__(64) void ring_signal_value(uint32_t* flag, uint32_t epoch) {
  if (threadIdx.x == 0) __hip_atomic_store(flag, epoch, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ __launch_bounds__(64) void ring_epoch(uint32_t* epoch) {
  if (threadIdx.x == 0) {
    const uint32_t e = *epoch + 1u;
    *epoch = e ? e : 1u;  // a zeroed flag never reads as done
  }
}

__global__ __launch_bounds__(kThreads) void poison_fill(uint4* p, int64_t n) {
  const uint4 nan4 = make_uint4(0xffffffffu, 0xffffffffu, 0xffffffffu, 0xffffffffu);
  for (int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x; i < n; i += int64_t(gridDim.x) * kThreads)
    p[i] = nan4;
}

// One lane per 4 head-dim values; the head_dim/4 lanes of one (row, head)
// are consecutive and lie inside one wavefront (head_dim/4 divides 64 and the
// loop stride is a multiple of 64), so every lane has read the old lse_acc
// before the lane with d4 == 0 overwrites it.
__global__ __launch_bounds__(kThreads) void lse_merge(MergeArgs a) {
  const int d4n = a.head_dim / 4;
  const int64_t per_row = int64_t(a.heads) * d4n;
  const int64_t total = int64_t(a.seg_len[0] + (a.nseg > 1 ? a.seg_len[1] : 0)) * per_row;
  for (int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x; i < total; i += int64_t(gridDim.x) * kThreads) {
    int64_t rr = i / per_row;
    const int64_t rem = i % per_row;
    const int h = int(rem / d4n), d4 = int(rem % d4n);
    const int64_t lrow = rr < a.seg_len[0] ? a.seg_start[0] + rr : a.seg_start[1] + (rr - a.seg_len[0]);
    const int64_t li = int64_t(h) * a.n_rows_total + lrow;
    const float ls = a.lse_s[li];
    const float la = a.lse_acc[li];
    const int64_t oi = (lrow * a.heads + h) * a.head_dim + 4 * d4;
    if (ls == -INFINITY) continue;  // nothing to fold in
    float wa = 0.f, ws = 1.f, L = ls;
    if (la != -INFINITY) {
      const float mx = fmaxf(la, ls);
      L = mx + log1pf(expf(-fabsf(la - ls)));
      wa = expf(la - L);
      ws = expf(ls - L);
    }
    const float4 os = *reinterpret_cast<const float4*>(a.o_s + oi);
    float4 r = make_float4(ws * os.x, ws * os.y, ws * os.z, ws * os.w);
    if (wa != 0.f) {
      const float4 oa = *reinterpret_cast<const float4*>(a.o_acc + oi);
      r.x += wa * oa.x;
      r.y += wa * oa.y;
      r.z += wa * oa.z;
      r.w += wa * oa.w;
    }
    *reinterpret_cast<float4*>(a.o_acc + oi) = r;
    if (d4 == 0) a.lse_acc[li] = L;
  }
}

__global__ __launch_bounds__(kThreads) void finalize_rows(FinalizeArgs a) {
  const int d4n = a.head_dim / 4;
  const int64_t per_row = int64_t(a.heads) * d4n;
  const int64_t total = int64_t(a.seg_len[0] + (a.nseg > 1 ? a.seg_len[1] : 0)) * per_row;
  for (int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x; i < total; i += int64_t(gridDim.x) * kThreads) {
    const int64_t rr = i / per_row;
    const int64_t rem = i % per_row;
    const int h = int(rem / d4n), d4 = int(rem % d4n);
    const bool second = rr >= a.seg_len[0];
    const int64_t off = second ? rr - a.seg_len[0] : rr;
    const int64_t lrow = (second ? a.seg_start[1] : a.seg_start[0]) + off;
    const int64_t grow = (second ? a.seg_global[1] : a.seg_global[0]) + off;
    const float4 o = *reinterpret_cast<const float4*>(a.acc_o + (lrow * a.heads + h) * a.head_dim + 4 * d4);
    const int64_t gi = (grow * a.heads + h) * a.head_dim + 4 * d4;
    if (a.out_f32) {
      *reinterpret_cast<float4*>(static_cast<float*>(a.out) + gi) = o;
    } else {
      typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
      bf16x4 b;
      b[0] = static_cast<__bf16>(o.x);
      b[1] = static_cast<__bf16>(o.y);
      b[2] = static_cast<__bf16>(o.z);
      b[3] = static_cast<__bf16>(o.w);
      *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(a.out) + gi) = b;
    }
    if (d4 == 0) a.lse[int64_t(h) * a.seq_len + grow] = a.acc_lse[int64_t(h) * a.n_loc + lrow];
  }
}

__global__ __launch_bounds__(kThreads) void fill_words(uint32_t* p, int64_t n, uint32_t value) {
  for (int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x; i < n; i += int64_t(gridDim.x) * kThreads) p[i] = value;
}

unsigned grid_for(int64_t work_items, int64_t per_block, unsigned cap) {
  int64_t g = (work_items + per_block - 1) / per_block;
  if (g < 1) g = 1;
  if (g > cap) g = cap;
  return unsigned(g);
}

}  // namespace

hipError_t launch_layout(const LayoutArgs& a, int max_blocks, hipStream_t stream) {
  const int64_t rows = int64_t(a.rank_count) * a.n_loc;
  const unsigned cap = max_blocks > 0 ? unsigned(max_blocks) : 65536u;
  const dim3 grid(grid_for(rows, 1, cap), unsigned(a.ntensors));
  layout_copy<<<grid, kThreads, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_ulysses(const UlyssesArgs& a, hipStream_t stream) {
  const int64_t rows = int64_t(a.cp) * a.seq_len;
  const int64_t run = a.heads / a.cp * a.head_vec;
  const int64_t rpw = run < kThreads ? kThreads / run : 1;  // rows per workgroup pass
  ulysses_copy<<<grid_for(rows, rpw, 65536u), kThreads, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_recv(const RecvArgs& a, int blocks, hipStream_t stream) {
  int64_t total = 0;
  for (int i = 0; i < a.n; ++i) total += a.vec[i];
  if (total == 0) return hipSuccess;
  const unsigned cap = blocks > 0 ? unsigned(blocks) : 65536u;
  recv_copy<<<grid_for(total, 64 * 2, cap), 64, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_ring_signal(uint32_t* flag, const uint32_t* epoch, hipStream_t stream) {
  ring_signal<<<1, 64, 0, stream>>>(flag, epoch);
  return hipGetLastError();
}

hipError_t launch_ring_signal_value(uint32_t* flag, uint32_t epoch, hipStream_t stream) {
  ring_signal_value<<<1, 64, 0, stream>>>(flag, epoch);
  return hipGetLastError();
}

hipError_t launch_ring_epoch(uint32_t* epoch, hipStream_t stream) {
  ring_epoch<<<1, 64, 0, stream>>>(epoch);
  return hipGetLastError();
}

// Fill words with a value (a kernel, so that it may sit in a captured graph).
hipError_t launch_fill_words(void* ptr, int64_t words, uint32_t value, hipStream_t stream) {
  if (words <= 0) return hipSuccess;
  fill_words<<<grid_for(words, kThreads, 1024u), kThreads, 0, stream>>>(static_cast<uint32_t*>(ptr), words, value);
  return hipGetLastError();
}

hipError_t launch_poison(void* ptr, int64_t bytes, hipStream_t stream) {
  const int64_t n = bytes / 16;
  poison_fill<<<grid_for(n, kThreads, 8192u), kThreads, 0, stream>>>(static_cast<uint4*>(ptr), n);
  return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t stream) {
  const int64_t total = int64_t(a.seg_len[0] + (a.nseg > 1 ? a.seg_len[1] : 0)) * a.heads * (a.head_dim / 4);
  lse_merge<<<grid_for(total, kThreads, 16384u), kThreads, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_finalize(const FinalizeArgs& a, hipStream_t stream) {
  const int64_t total = int64_t(a.seg_len[0] + (a.nseg > 1 ? a.seg_len[1] : 0)) * a.heads * (a.head_dim / 4);
  finalize_rows<<<grid_for(total, kThreads, 16384u), kThreads, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace cpattn
