// C ABI of libcpattn.so and the one-GPU ring step scheduler.
//
// The ring ("Sequence Parallelism IV: Megatron Context Parallel and
// Load-Balanced Rings", section 4 "What Actually Moves" and section 5
// "Overlap: More Than One Stream"): the rank's queries stay put while the K/V
// of source (r - s) mod cp arrives at step s.  On one GPU the arrival is a
// device-to-device copy into one of two receive slots, issued on a side
// stream one step ahead so it runs under the current step's attention; the
// softmax-state correction either runs in the attention kernel's epilogue
// (default) or as a separate LSE-merge kernel on its own stream, so it does
// not serialize the ring steps.  HIP events carry the cross-stream edges:
//   copy(s+1 -> slot (s+1)&1) waits attn_done[(s+1)&1]   (step s-1 released it)
//   attn(s, slot s&1)          waits recv_done[s&1]
//   attn(s) -> part[s&1]       waits merge_done[s&1]      (separate merge only)
//   merge(s)                   waits attn_done[s&1]
#include <hip/hip_runtime.h>

#include <algorithm>
#include <array>
#include <cmath>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "cp_attn.h"
#include "kernels.h"
#include "plan.h"

struct cp_attn_plan_s {
  cpattn::Plan* p;
};

namespace cpattn {

struct DeviceState {
  int device = -1;
  hipStream_t copy = nullptr;
  hipStream_t merge = nullptr;
  bool own_copy = false, own_merge = false;
  bool events_ready = false;
  hipEvent_t start = nullptr, merge_join = nullptr;
  hipEvent_t recv_done[2] = {nullptr, nullptr};
  hipEvent_t attn_done[2] = {nullptr, nullptr};
  hipEvent_t merge_done[2] = {nullptr, nullptr};
  void* ws = nullptr;
  int64_t ws_bytes = 0;
  bool own_ws = false;
  std::vector<hipEvent_t> t0, t1;  // per (rank, step) timing events
  std::vector<int> timed;          // 1 if (rank, step) was timed by the last call
  // graph mode: the last recorded forward and what it was recorded for
  hipStream_t capture = nullptr;
  hipGraphExec_t graph = nullptr;
  std::vector<intptr_t> graph_key;
  int64_t doc_uploaded = -1;  // plan doc_version whose document table the workspace holds
  int cus = 0;             // compute units of the device
  // work counters (CP_ATTN_OPT_COUNTERS): key tiles computed per (rank, step)
  unsigned long long* tile_cnt = nullptr;
  std::vector<int> counted;  // 1 if (rank, step) was counted by the last call
  // lockstep full forward (CP_ATTN_OPT_LOCKSTEP): every rank's receive slots
  // and running state, the step-argument table and its workgroup ranges
  char* ls_ws = nullptr;
  int64_t ls_bytes = 0;
  void* ls_host = nullptr;         // pinned staging of the table
  hipEvent_t ls_uploaded = nullptr;
  std::vector<intptr_t> ls_key;    // what the uploaded table was built for
  // fused ring (CP_ATTN_OPT_FUSED_RING): receive slots of steps 1 .. P-1 (all
  // the K slots, then all the V slots), a flag per step (zeroed once), every
  // rank's key runs (uploaded once) with each rank's two row ranges, the
  // epoch of the last call and the host-visible time-out word
  char* fr_slots = nullptr;
  int64_t fr_slots_bytes = 0;
  uint32_t* fr_flags = nullptr;
  RingRun* fr_runs = nullptr;
  std::vector<SegArgs> fr_segs;  // [rank * 2 + i]: late rows, then early rows (run0 set)
  // key split of the fused launch: [rank * 4 + i], seg[0..3] of the launch
  // (part 0 of late and early rows, then their part 1), used where fr_split[rank]
  std::vector<SegArgs> fr_split_segs;
  std::vector<uint8_t> fr_split;
  std::vector<uint8_t> fr_need;  // [rank * cp + step]: a run of the rank reads step's slot
  // second lane of cp_attn_full_forward's fused ranks (odd ranks): its own
  // compute and copy streams, slots, flags and events, so that one rank's
  // launch runs beside the next one's
  hipStream_t fl_comp = nullptr, fl_copy = nullptr;
  char* fl_slots = nullptr;
  int64_t fl_slots_bytes = 0;
  uint32_t* fl_flags = nullptr;
  char* fl_split = nullptr;  // key split's partial outputs, LSEs and counters of the second lane
  hipEvent_t fl_enter = nullptr, fl_join = nullptr, fl_start = nullptr, fl_recv[2] = {nullptr, nullptr};
  int fr_nseg = 2;               // row ranges per rank: 2 zigzag (late, early), 1 contiguous
  bool fr_lanes = false;         // full forward: two lanes (short launches only)
  // calls recorded into a graph use their own flags, whose word 0 a kernel
  // advances at the start of each replay; other calls are numbered by the
  // host (fr_host_epoch) and leave word 0 of their flags at zero
  uint32_t* fr_gflags = nullptr;
  uint32_t fr_host_epoch = 0;
  bool fr_ok = false;            // the plan's runs are whole tiles (built once)
  bool fr_built = false;
  uint32_t* fr_err = nullptr;
  uint32_t* fr_err_dev = nullptr;
  int fr_last = 0;  // the last forward call ran every rank it computed as one fused launch
};

namespace {

thread_local std::string g_err;

int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

#define CPA_HIP(call)                                                                   \
  do {                                                                                  \
    hipError_t e_ = (call);                                                             \
    if (e_ != hipSuccess) return fail(CP_ATTN_EHIP, std::string(#call) + ": " + hipGetErrorString(e_)); \
  } while (0)

struct WsLayout {
  int64_t slot_k[2], slot_v[2], acc_o, acc_lse, part_o[2], part_lse[2], split_cnt, doc, total;
  int64_t kv_bytes, o_bytes, lse_bytes, cnt_bytes, doc_bytes;
};

// row tiles of the key-split kernel (256 rows) over a step's two segments,
// one counter per (row tile, head)
int64_t split_counters(const Plan& p) { return (p.n_loc / 256 + 2) * p.heads; }

int64_t align256(int64_t x) { return (x + 255) & ~int64_t(255); }

WsLayout ws_layout(const Plan& p) {
  WsLayout w{};
  w.kv_bytes = p.n_loc * p.heads * p.head_dim * p.elem_bytes();
  w.o_bytes = p.n_loc * p.heads * p.head_dim * 4;
  w.lse_bytes = int64_t(p.heads) * p.n_loc * 4;
  int64_t off = 0;
  auto take = [&](int64_t n) {
    const int64_t at = off;
    off += align256(n);
    return at;
  };
  for (int b = 0; b < 2; ++b) {
    w.slot_k[b] = take(w.kv_bytes);
    w.slot_v[b] = take(w.kv_bytes);
  }
  w.acc_o = take(w.o_bytes);
  w.acc_lse = take(w.lse_bytes);
  for (int b = 0; b < 2; ++b) {
    w.part_o[b] = take(w.o_bytes);
    w.part_lse[b] = take(w.lse_bytes);
  }
  w.cnt_bytes = split_counters(p) * 4;
  w.split_cnt = take(w.cnt_bytes);
  w.doc_bytes = p.seq_len * 8;  // document table: [start, end) per position, int32
  w.doc = take(w.doc_bytes);
  w.total = off;
  return w;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Device, streams and events of the plan; with need_ws also the workspace
// (allocated on first use unless the caller gave one) and the document table
// in it.  The single-launch forwards (all-gather, Ulysses) need the workspace
// only for the document table.
int ensure_device(Plan& p, bool need_ws = true) {
  DeviceState& d = *p.dev;
  int dev = 0;
  CPA_HIP(hipGetDevice(&dev));
  if (d.device >= 0 && d.device != dev)
    return fail(CP_ATTN_EINVAL, "plan was first used on another device");
  d.device = dev;
  if (!d.events_ready) {
    CPA_HIP(hipEventCreateWithFlags(&d.start, hipEventDisableTiming));
    CPA_HIP(hipEventCreateWithFlags(&d.merge_join, hipEventDisableTiming));
    for (int b = 0; b < 2; ++b) {
      CPA_HIP(hipEventCreateWithFlags(&d.recv_done[b], hipEventDisableTiming));
      CPA_HIP(hipEventCreateWithFlags(&d.attn_done[b], hipEventDisableTiming));
      CPA_HIP(hipEventCreateWithFlags(&d.merge_done[b], hipEventDisableTiming));
    }
    d.events_ready = true;
  }
  if (!d.copy) {
    CPA_HIP(hipStreamCreateWithFlags(&d.copy, hipStreamNonBlocking));
    d.own_copy = true;
  }
  if (!d.merge) {
    CPA_HIP(hipStreamCreateWithFlags(&d.merge, hipStreamNonBlocking));
    d.own_merge = true;
  }
  if (!d.cus) CPA_HIP(hipDeviceGetAttribute(&d.cus, hipDeviceAttributeMultiprocessorCount, dev));
  if (!need_ws) return CP_ATTN_OK;
  const WsLayout w = ws_layout(p);
  if (d.ws && d.ws_bytes < w.total) {
    if (!d.own_ws) return fail(CP_ATTN_ENOWORKSPACE, "caller workspace smaller than cp_attn_workspace_bytes");
    CPA_HIP(hipFree(d.ws));
    d.ws = nullptr;
    d.ws_bytes = 0;
  }
  if (!d.ws) {
    if (hipMalloc(&d.ws, size_t(w.total)) != hipSuccess) {
      d.ws = nullptr;
      return fail(CP_ATTN_ENOWORKSPACE, "hipMalloc of the workspace failed");
    }
    d.ws_bytes = w.total;
    d.own_ws = true;
    d.doc_uploaded = -1;
  }
  if (!p.doc_starts.empty() && d.doc_uploaded != p.doc_version) {
    // the document table of the current list: once per list and workspace,
    // synchronously (kernels still queued may read the old table)
    std::vector<int32_t> tab(size_t(p.seq_len) * 2);
    for (size_t dd = 0; dd < p.doc_starts.size(); ++dd) {
      const int64_t b = p.doc_starts[dd], e = dd + 1 < p.doc_starts.size() ? p.doc_starts[dd + 1] : p.seq_len;
      for (int64_t i = b; i < e; ++i) {
        tab[size_t(i) * 2] = int32_t(b);
        tab[size_t(i) * 2 + 1] = int32_t(e);
      }
    }
    CPA_HIP(hipDeviceSynchronize());
    CPA_HIP(hipMemcpy(static_cast<char*>(d.ws) + w.doc, tab.data(), size_t(w.doc_bytes), hipMemcpyHostToDevice));
    d.doc_uploaded = p.doc_version;
  }
  if (p.opt_counters && !d.tile_cnt)
    CPA_HIP(hipMalloc(&d.tile_cnt, size_t(p.cp) * p.cp * sizeof(unsigned long long)));
  if (p.opt_step_timing && d.t0.empty()) {
    const size_t n = size_t(p.cp) * p.cp;
    d.t0.assign(n, nullptr);
    d.t1.assign(n, nullptr);
    for (size_t i = 0; i < n; ++i) {
      CPA_HIP(hipEventCreate(&d.t0[i]));
      CPA_HIP(hipEventCreate(&d.t1[i]));
    }
  }
  return CP_ATTN_OK;
}

// What one forward call runs with: the workspace base and the schedule.  A
// plain call takes both from the plan; the no-allocation entry point runs the
// same steps on the library's static scratch, on the caller's stream only.
struct RunCfg {
  char* ws = nullptr;      // workspace base (ws_layout offsets apply)
  bool serial = false;     // every step on the caller's stream, no events
  int recv = 0;            // CP_ATTN_OPT_RECV in effect
  int recv_blocks = 256;   // CP_ATTN_OPT_RECV_BLOCKS in effect beside a step launch
  int recv_blocks_fused = 1024;  // and beside the fused ring's one launch
  int fused_ring = 0;      // CP_ATTN_OPT_FUSED_RING in effect
  bool capturing = false;  // the calls are being recorded into a graph
  bool counters = false;   // device work counters (plan-owned buffer)
  bool timing = false;     // per-step timing events
  bool poison = false;     // NaN-fill consumed buffers
};

RunCfg plan_cfg(const Plan& p, bool capturing) {
  RunCfg c;
  c.ws = static_cast<char*>(p.dev->ws);
  c.serial = p.opt_serialize != 0;
  c.recv = p.opt_recv;
  // automatic receive grid: beside one step launch, 256 workgroups leave it
  // its compute units; the fused launch's later steps wait for the receives,
  // which then need the wider grid to keep ahead (32k/cp8: the late ranks'
  // calls 1.10 ms at 256, 0.96 at 1024, as rank 0's)
  c.recv_blocks = p.opt_recv_blocks < 0 ? 256 : p.opt_recv_blocks;
  c.recv_blocks_fused = p.opt_recv_blocks < 0 ? 1024 : p.opt_recv_blocks;
  c.counters = p.opt_counters != 0;
  c.timing = p.opt_step_timing != 0 && !capturing;
  c.poison = p.opt_poison != 0;
  c.fused_ring = p.opt_fused_ring;
  c.capturing = capturing;
  return c;
}

// The K and V rows of ring source `src` (its local order) are one (contiguous)
// or two (zigzag) token ranges of the natural-order tensors; receiving them
// into slot b is two or four linear copies.  Only real rows are received: a
// chunk's pad rows (and a chunk of pad only) are not copied, and the kernels
// never read past the source's real keys.
// The step kernels address K/V with 32-bit byte offsets from one base.  The
// natural-order tensors are read in place at step 0 only while they span at
// most 4 GiB; beyond that step 0, like every later step, reads the rank's own
// chunks from receive slot 0, filled by one copy before it.
bool kv_beyond_32bit(const Plan& p) {
  return p.seq_len * p.heads * p.head_dim * p.elem_bytes() > int64_t(UINT32_MAX);
}

RecvArgs recv_ranges_to(const Plan& p, char* dk, char* dv, const void* k, const void* v, int src) {
  const int64_t row_bytes = int64_t(p.heads) * p.head_dim * p.elem_bytes();
  const int nch = p.layout == 1 ? 2 : 1;
  const int64_t ch_bytes = p.chunk * row_bytes;
  RecvArgs ra{};
  for (int c = 0; c < nch; ++c) {
    const int64_t g = p.chunk_of(src, c) * ch_bytes;
    const int64_t bytes = p.valid_in_chunk(p.chunk_of(src, c)) * row_bytes;
    if (bytes == 0) continue;
    ra.src[ra.n] = static_cast<const char*>(k) + g;
    ra.dst[ra.n] = dk + c * ch_bytes;
    ra.vec[ra.n++] = bytes / 16;
    ra.src[ra.n] = static_cast<const char*>(v) + g;
    ra.dst[ra.n] = dv + c * ch_bytes;
    ra.vec[ra.n++] = bytes / 16;
  }
  return ra;
}

RecvArgs recv_ranges(const Plan& p, char* ws, const void* k, const void* v, int src, int b) {
  const WsLayout w = ws_layout(p);
  return recv_ranges_to(p, ws + w.slot_k[b], ws + w.slot_v[b], k, v, src);
}

// Side-stream receive of ring source `src` into slot b.  `alone`: no step
// kernel runs beside it (serial order, or a step that launches nothing), so
// the copy takes the whole chip instead of the few workgroups that leave the
// step kernel its compute units.
int recv_kv(const Plan& p, const RunCfg& c, const void* k, const void* v, int src, int b, bool alone,
            hipStream_t s) {
  const RecvArgs ra = recv_ranges(p, c.ws, k, v, src, b);
  if (c.recv == 1) {
    for (int i = 0; i < ra.n; ++i)
      CPA_HIP(hipMemcpyAsync(ra.dst[i], ra.src[i], size_t(ra.vec[i] * 16), hipMemcpyDeviceToDevice, s));
    return CP_ATTN_OK;
  }
  CPA_HIP(launch_recv(ra, alone ? 0 : c.recv_blocks, s));
  return CP_ATTN_OK;
}

// Whether step s's attention kernel itself receives step s+1's K/V (mode 2
// at every step; mode 3 from step 1 on, step 0's receive going through the
// copy stream), and whether step s's receive runs on the copy stream.
bool kernel_recv(const Plan& p, const RunCfg& c, int s) {
  if (s + 1 >= p.cp || !attn_does_recv(p.dtype == CP_ATTN_BF16, p.head_dim)) return false;
  return c.recv == 2 || (c.recv == 3 && s >= 1);
}
bool side_recv(const Plan& p, const RunCfg& c, int s) { return s + 1 < p.cp && !kernel_recv(p, c, s); }

// Document masks of a launch whose keys are source j's local buffer (j < 0:
// the identity map, keys at their own positions).  A is StepArgs or BwdArgs.
template <typename A>
void set_doc(const Plan& p, const char* ws, A& a, int j) {
  if (p.doc_starts.empty()) return;
  a.doc = reinterpret_cast<const int32_t*>(ws + ws_layout(p).doc);
  if (j < 0) {
    a.kpos_lo = 0;
    a.kpos_hi = 0;
    a.kpos_split = a.n_loc;
  } else {
    a.kpos_lo = int32_t(p.chunk_of(j, 0) * p.chunk);
    a.kpos_hi = p.layout == 1 ? int32_t(p.chunk_of(j, 1) * p.chunk) : 0;
    a.kpos_split = int32_t(p.layout == 1 ? p.chunk : p.n_loc);
  }
}

// Key split: when a step's workgroups would fill at most half the GPU, each
// full segment's row tiles take two workgroups, one per half of the keys (the
// partial buffers of the separate merge mode hold the parts).  Returns the
// ksplit factor (1 or 2) of segment i of (r, s).
int seg_ksplit(const Plan& p, int r, int s, int i, bool lockstep = false) {
  if (lockstep) return 1;  // every rank's step fills the GPU together, and the split buffers are per rank
  const StepDesc& sd = p.step(r, s);
  const bool bf16 = p.dtype == CP_ATTN_BF16;
  if (!p.opt_ksplit || p.opt_merge == 1 || !p.doc_starts.empty() || !attn_splits_keys(bf16, p.head_dim)) return 1;
  const int bm = attn_bf16_block_m(p.head_dim);
  int64_t wgs = 0;
  for (int t = 0; t < sd.nseg; ++t) wgs += (sd.seg[t].q_len + bm - 1) / bm * p.heads;
  if (2 * wgs > p.dev->cus) return 1;
  const Segment& g = sd.seg[i];
  // the kernel keeps a split row tile's parts in 128 KiB slots of the
  // partial buffers, one per (256-row tile of the local rows, head)
  return !g.diag && g.kv_full >= 16 * 64 && g.q_start % 256 == 0 && p.n_loc % 256 == 0 ? 2 : 1;
}

bool rank_splits(const Plan& p, int r) {
  for (int s = 0; s < p.cp; ++s)
    for (int i = 0; i < p.step(r, s).nseg; ++i)
      if (seg_ksplit(p, r, s, i) > 1) return true;
  return false;
}

// The arguments of step (r, s).  Step 0 reads the rank's own K/V in place
// (the rank holds them; nothing is received); later steps read receive slot
// b.  ws: the workspace holding the rank's slots and running state; the
// document table is always the plan's (dws).  lockstep: every rank's step in
// one launch (no key split, no in-kernel receive).
StepArgs make_step_args(Plan& p, const RunCfg& c, const void* q, const void* k, const void* v, void* out, float* lse,
                        int r, int s, int b, char* ws, const char* dws, bool lockstep) {
  DeviceState& d = *p.dev;
  const WsLayout w = ws_layout(p);
  const StepDesc& sd = p.step(r, s);
  const bool bf16 = p.dtype == CP_ATTN_BF16;
  const int bm = bf16 ? attn_bf16_block_m(p.head_dim) : attn_f32_block_m();
  StepArgs a{};
  a.q = q;
  const int32_t split = int32_t(p.layout == 1 ? p.chunk : p.n_loc);
  if (s == 0 && !kv_beyond_32bit(p)) {  // the rank's own chunks, read in place
    a.k = k;
    a.v = v;
    a.kv_bytes = p.seq_len * p.heads * p.head_dim * p.elem_bytes();
    a.kv_lo = int32_t(p.chunk_of(r, 0) * p.chunk);
    a.kv_hi = p.layout == 1 ? int32_t(p.chunk_of(r, 1) * p.chunk) : 0;
    a.kv_split = split;
  } else {
    a.k = ws + w.slot_k[b];
    a.v = ws + w.slot_v[b];
    a.kv_bytes = w.kv_bytes;
    a.kv_lo = 0;
    a.kv_hi = split;
    a.kv_split = split;
  }
  a.acc_o = reinterpret_cast<float*>(ws + w.acc_o);
  a.acc_lse = reinterpret_cast<float*>(ws + w.acc_lse);
  a.part_o = reinterpret_cast<float*>(ws + w.part_o[b]);
  a.part_lse = reinterpret_cast<float*>(ws + w.part_lse[b]);
  a.out = out;
  a.lse = lse;
  a.seq_len = p.seq_len;
  a.n_loc = int32_t(p.n_loc);
  a.kv_valid = int32_t(p.valid_rows(sd.src));
  a.heads = p.heads;
  a.scale = 1.0f / std::sqrt(float(p.head_dim));
  a.scale_log2 = a.scale * 1.4426950408889634f;
  a.out_f32 = p.dtype == CP_ATTN_FP32;
  a.nseg = sd.nseg;
  a.total_tiles = 0;
  const bool separate = p.opt_merge == 1;
  for (int b = 0; b < 2; ++b) {
    a.split_o[b] = reinterpret_cast<float*>(ws + w.part_o[b]);
    a.split_lse[b] = reinterpret_cast<float*>(ws + w.part_lse[b]);
  }
  a.split_cnt = reinterpret_cast<int32_t*>(ws + w.split_cnt);
  for (int i = 0; i < sd.nseg; ++i) {
    const Segment& g = sd.seg[i];
    SegArgs& x = a.seg[i];
    x.q_global = g.q_global;
    x.q_start = int32_t(g.q_start);
    x.q_len = int32_t(g.q_len);
    x.kv_full = int32_t(g.kv_full);
    x.diag = g.diag;
    const int32_t qt = int32_t((g.q_len + bm - 1) / bm);
    x.ksplit = seg_ksplit(p, r, s, i, lockstep);
    x.tiles = qt * x.ksplit;
    if (separate) {
      x.epi = g.first ? kEpiInit : kEpiPartial;
    } else {
      x.epi = (g.first ? kEpiInit : kEpiMerge) | (g.last ? kEpiFinal : 0);
    }
    a.total_tiles += x.tiles;
  }
  if (sd.nseg == 1) a.seg[1] = SegArgs{};
  // Workgroups are dispatched in segment order: the segment with the longer
  // rows goes first, so that (each segment already ordered longest row tile
  // first) the short tiles of the other fill in behind the long ones.  On a
  // rank's first step this pairs the long row tiles of the late chunk with
  // the short diagonal tiles of the early one on the same compute unit.
  if (sd.nseg == 2) {
    auto work = [](const SegArgs& x) { return int64_t(x.q_len) * (2 * int64_t(x.kv_full) + (x.diag ? x.q_len : 0)); };
    if (work(a.seg[1]) > work(a.seg[0])) std::swap(a.seg[0], a.seg[1]);
  }
  if (!lockstep && kernel_recv(p, c, s)) a.recv = recv_ranges(p, ws, k, v, p.step(r, s + 1).src, (s + 1) & 1);
  if (c.counters) a.tile_cnt = d.tile_cnt + size_t(r) * p.cp + s;
  set_doc(p, dws, a, sd.src);
  return a;
}

int launch_step(Plan& p, const RunCfg& c, const void* q, const void* k, const void* v, void* out, float* lse, int r,
                int s, int b, hipStream_t st) {
  char* ws = c.ws;
  const StepDesc& sd = p.step(r, s);
  const bool bf16 = p.dtype == CP_ATTN_BF16;
  if (sd.nseg == 0) {
    // no query row of this rank sees the step's keys; the receive still happens
    if (kernel_recv(p, c, s)) CPA_HIP(launch_recv(recv_ranges(p, ws, k, v, p.step(r, s + 1).src, (s + 1) & 1), 0, st));
    return CP_ATTN_OK;
  }
  const StepArgs a = make_step_args(p, c, q, k, v, out, lse, r, s, b, ws, ws, false);
  const hipError_t e = bf16 ? launch_attn_bf16(a, p.head_dim, st) : launch_attn_f32(a, p.head_dim, st);
  if (e != hipSuccess) return fail(CP_ATTN_EHIP, std::string("attention launch: ") + hipGetErrorString(e));
  return CP_ATTN_OK;
}

// Separate-merge mode: fold part[b] of step (r, s) into the running state.
int launch_step_merge(Plan& p, char* ws, int r, int s, int b, hipStream_t ms) {
  const WsLayout w = ws_layout(p);
  const StepDesc& sd = p.step(r, s);
  MergeArgs m{};
  m.o_s = reinterpret_cast<const float*>(ws + w.part_o[b]);
  m.lse_s = reinterpret_cast<const float*>(ws + w.part_lse[b]);
  m.o_acc = reinterpret_cast<float*>(ws + w.acc_o);
  m.lse_acc = reinterpret_cast<float*>(ws + w.acc_lse);
  m.n_rows_total = p.n_loc;
  m.heads = p.heads;
  m.head_dim = p.head_dim;
  for (int i = 0; i < sd.nseg; ++i) {
    if (sd.seg[i].first) continue;  // written straight into the state
    m.seg_start[m.nseg] = int32_t(sd.seg[i].q_start);
    m.seg_len[m.nseg] = int32_t(sd.seg[i].q_len);
    ++m.nseg;
  }
  if (m.nseg == 0) return CP_ATTN_OK;
  CPA_HIP(launch_merge(m, ms));
  return CP_ATTN_OK;
}

int launch_rank_finalize(Plan& p, const char* ws, void* out, float* lse, int r, hipStream_t st) {
  const WsLayout w = ws_layout(p);
  FinalizeArgs f{};
  f.acc_o = reinterpret_cast<const float*>(ws + w.acc_o);
  f.acc_lse = reinterpret_cast<const float*>(ws + w.acc_lse);
  f.out = out;
  f.lse = lse;
  f.seq_len = p.seq_len;
  f.n_loc = int32_t(p.n_loc);
  f.heads = p.heads;
  f.head_dim = p.head_dim;
  f.out_f32 = p.dtype == CP_ATTN_FP32;
  const int nch = p.layout == 1 ? 2 : 1;
  for (int c = 0; c < nch; ++c) {  // real rows only
    const int64_t len = p.valid_in_chunk(p.chunk_of(r, c));
    if (len == 0) continue;
    f.seg_start[f.nseg] = int32_t(c * p.chunk);
    f.seg_len[f.nseg] = int32_t(len);
    f.seg_global[f.nseg] = p.global_row(r, c * p.chunk);
    ++f.nseg;
  }
  if (f.nseg == 0) return CP_ATTN_OK;
  CPA_HIP(launch_finalize(f, st));
  return CP_ATTN_OK;
}

#define CPA_TRY(x)                \
  do {                            \
    const int rc_ = (x);          \
    if (rc_ != CP_ATTN_OK) return rc_; \
  } while (0)

// ---- fused ring ----
// Every ring step of a rank in one launch of the step kernel: each row tile
// takes the keys of all its steps in turn with the running max and sum in
// registers (the exact merge of "Sequence Parallelism IV: Megatron Context
// Parallel and Load-Balanced Rings", section 4, carried across steps instead
// of stored between launches) and writes its output once.  The receives of
// steps 1 .. P-1 still arrive one by one on the copy stream ("Sequence
// Parallelism IV", section 5, "Overlap: More Than One Stream"), each into a
// slot of its own and followed by a one-thread kernel that stores the call's
// epoch to the step's flag; a workgroup waits for that flag before loading
// any key of the step.  Served for bf16 head_dim 128, zigzag (two row ranges)
// and contiguous (one) layouts, causal or bidirectional, without padding,
// chunks of whole 64-key tiles, the fused merge and
// the copy-kernel receive, outside the serial, counter and poison modes,
// without document masks, while the own K/V and the slots each span at most
// 4 GiB.  Step timing reports the launch under step 0.  The call's epoch
// lives in device memory (flag word 0), advanced by a kernel at the start of
// the call, so that a recorded graph's replays each wait for their own
// receives.

constexpr int kRingPolls = 1 << 18;  // polls (each a coherent load and a short sleep, ~0.2-2 us) before a wait gives up

bool fused_ring_served(const Plan& p, const RunCfg& c) {
  if (!c.fused_ring || c.serial || c.recv != 0 || c.counters || c.poison) return false;
  if (p.dtype != CP_ATTN_BF16 || p.head_dim != 128 || p.opt_merge != 0) return false;
  if (!p.doc_starts.empty() || p.cp < 2 || kv_beyond_32bit(p) || p.padded_len != p.seq_len) return false;
  if (int64_t(p.cp - 1) * ws_layout(p).kv_bytes > int64_t(UINT32_MAX)) return false;
  return p.dev->fr_ok || !p.dev->fr_built;  // (the run check needs the table: built at the first call)
}

// The key runs of rank r's row range [R0, R0 + chunk): the keys its
// segments see at each step, in step order (the rank's own chunks read in
// place at step 0, slot s at step s >= 1), then its causal diagonal (step 0).
// Returns false if a run is not a whole number of 64-key tiles or a step's
// segments do not cover the range whole.
bool ring_runs(const Plan& p, int r, int64_t R0, std::vector<RingRun>& runs, SegArgs& sa) {
  const int64_t C = p.chunk;
  int64_t key = 0, diag_lo = -1;
  auto own_row = [&](int64_t kk) { return kk < C ? p.chunk_of(r, 0) * C + kk : p.chunk_of(r, 1) * C + (kk - C); };
  auto add = [&](int64_t n, int64_t row, int buf, int step) {
    if (n <= 0) return true;
    if (n % 64) return false;
    runs.push_back(RingRun{int32_t(key + n), int32_t(row - key), buf, step});
    key += n;
    return true;
  };
  for (int s = 0; s < p.cp; ++s) {
    const StepDesc& sd = p.step(r, s);
    for (int i = 0; i < sd.nseg; ++i) {
      const Segment& g = sd.seg[i];
      if (g.q_start + g.q_len <= R0 || g.q_start >= R0 + C) continue;  // not these rows
      if (g.q_start > R0 || g.q_start + g.q_len < R0 + C) return false;  // part of them
      if (s == 0) {
        // the own buffer's two chunks are apart in the natural order
        if (!add(std::min(g.kv_full, C), own_row(0), 0, -1)) return false;
        if (!add(g.kv_full - C, own_row(C), 0, -1)) return false;
      } else if (!add(g.kv_full, int64_t(s - 1) * p.n_loc, 1, s)) {
        return false;
      }
      if (g.diag) {
        if (s != 0 || g.q_start != R0) return false;
        diag_lo = g.kv_full;
      }
    }
  }
  sa = SegArgs{};
  sa.q_start = int32_t(R0);
  sa.q_len = int32_t(C);
  sa.q_global = p.global_row(r, R0);
  sa.kv_full = int32_t(key);
  sa.diag = diag_lo >= 0 ? 1 : 0;
  if (sa.diag && !add(C, own_row(diag_lo), 0, -1)) return false;
  sa.epi = kEpiInit | kEpiFinal;
  const int bm = attn_bf16_block_m(128);
  sa.tiles = int32_t((C + bm - 1) / bm);
  sa.ksplit = 1;
  return !runs.empty();
}

// Key split of a segment's run list: part 0 takes the first half of every
// full run, part 1 the second halves and then the diagonal run (the last run
// when sa.diag), each in a key space of its own from 0.  The halves keep the
// step order, so each part waits for the receives in the order they land.
// Returns false if a full run's half is not a whole number of 64-key tiles.
bool split_ring_runs(const std::vector<RingRun>& runs, const SegArgs& sa, std::vector<RingRun> part[2]) {
  int64_t beg = 0, key[2] = {0, 0};
  const size_t nfull = runs.size() - (sa.diag ? 1 : 0);
  for (size_t i = 0; i < runs.size(); ++i) {
    const RingRun& u = runs[i];
    const int64_t n = u.end - beg;
    if (i < nfull) {
      if (n % 128) return false;
      for (int pp = 0; pp < 2; ++pp) {
        const int64_t first = beg + pp * (n / 2);  // the half's first key in the segment's key space
        part[pp].push_back(RingRun{int32_t(key[pp] + n / 2), int32_t(first + u.delta - key[pp]), u.buf, u.step});
        key[pp] += n / 2;
      }
    } else {
      part[1].push_back(RingRun{int32_t(key[1] + n), int32_t(beg + u.delta - key[1]), u.buf, u.step});
    }
    beg = u.end;
  }
  return !part[0].empty();
}

// Estimated length, in 64-key tiles, of a fused launch whose segments have
// row tiles of the given key-tile counts (full and diagonal keys apart).
// Workgroups start in dispatch order (segment by segment, longest row tiles
// first, a split tile's parts side by side, every head of a tile together),
// one per compute unit.  The chip's clock is bound by its power: measured,
// every compute unit busy gives only about 1.4 times the throughput of half
// of them, so a workgroup runs at full speed while at most half the compute
// units are busy and at (half / busy)^0.5 of it beyond.  A workgroup adds a
// fixed cost of 16 tiles (prologue, first receive, epilogue), a split part 2
// more for the fold.  (Fitted to the rank calls of the 8192-token cp 4
// 32-head and the 16384-token cp 4 16-head workloads, within 4 %.)
double ring_launch_tiles(const std::vector<std::array<int64_t, 2>> tiles[2], const int split[2], int heads, int cus) {
  constexpr double kWg = 16.0, kFold = 2.0;
  std::vector<double> queue;
  for (int i = 0; i < 2; ++i)
    for (const auto& rt : tiles[i])
      for (int pp = 0; pp < split[i]; ++pp) {
        const double c = split[i] == 1 ? kWg + double(rt[0] + rt[1])
                                        : kWg + kFold + double(rt[0] / 2 + (pp ? rt[1] : 0));
        for (int h = 0; h < heads; ++h) queue.push_back(c);
      }
  std::vector<double> busy;  // work left of the running workgroups
  size_t next = 0;
  double t = 0.0;
  const double half = std::max(1, cus / 2);
  while (next < queue.size() || !busy.empty()) {
    while (next < queue.size() && int(busy.size()) < cus) busy.push_back(queue[next++]);
    const double n = double(busy.size());
    const double rate = n <= half ? 1.0 : std::sqrt(half / n);
    const double m = *std::min_element(busy.begin(), busy.end());
    t += m / rate;
    size_t k = 0;
    for (double b : busy)
      if (b - m > 1e-9) busy[k++] = b - m;
    busy.resize(k);
  }
  return t;
}

// The run table of every rank, uploaded once per plan (set-up, synchronous).
int ensure_fused_ring(Plan& p) {
  DeviceState& d = *p.dev;
  if (!d.fr_built) {
    d.fr_built = true;
    d.fr_ok = false;
    std::vector<RingRun> all;
    d.fr_segs.assign(size_t(p.cp) * 2, SegArgs{});
    d.fr_split_segs.assign(size_t(p.cp) * 4, SegArgs{});
    d.fr_split.assign(size_t(p.cp), 0);
    d.fr_need.assign(size_t(p.cp) * p.cp, 0);
    bool ok = true;
    const int bm = attn_bf16_block_m(128);
    // zigzag: the late rows first (causal: they see more keys), then the
    // early rows; contiguous: the rank's one chunk
    const int nr = p.layout == 1 ? 2 : 1;
    d.fr_nseg = nr;
    for (int r = 0; r < p.cp && ok; ++r) {
      const int64_t R0[2] = {nr == 2 ? p.chunk : 0, 0};
      std::vector<RingRun> runs[2];
      for (int i = 0; i < nr && ok; ++i) {
        SegArgs& sa = d.fr_segs[size_t(r) * 2 + i];
        ok = ring_runs(p, r, R0[i], runs[i], sa);
        sa.run0 = int32_t(all.size());
        all.insert(all.end(), runs[i].begin(), runs[i].end());
        for (const RingRun& u : runs[i])
          if (u.step > 0) d.fr_need[size_t(r) * p.cp + u.step] = 1;
      }
      if (!ok) break;
      // key split: where the launch would leave compute units idle (few
      // heads, or one segment's rows seeing most of the keys), a segment's
      // row tiles may take two workgroups each.  The split's fold keeps a
      // part in a 128 KiB slot per (256-row tile, head) of the workspace.
      if (bm != 256 || p.chunk % 256 || p.n_loc % 256) continue;
      // (a segment whose rows see only the diagonal, rank 0's early rows,
      // has nothing to split)
      std::vector<RingRun> halves[2][2];
      bool can[2];
      std::vector<std::array<int64_t, 2>> rt[2];
      for (int i = 0; i < 2; ++i) {
        const SegArgs& sa = d.fr_segs[size_t(r) * 2 + i];
        can[i] = split_ring_runs(runs[i], sa, halves[i]);
        for (int64_t t = sa.tiles - 1; t >= 0; --t)  // longest first
          rt[i].push_back({sa.kv_full / 64, sa.diag ? (t + 1) * bm / 64 : 0});
      }
      int best[2] = {1, 1};
      const int none[2] = {1, 1};
      const double base = ring_launch_tiles(rt, none, p.heads, d.cus);
      double best_len = base;
      for (int o = 1; o < 4; ++o) {
        const int sp[2] = {1 + (o & 1), 1 + (o >> 1)};
        if ((sp[0] > 1 && !can[0]) || (sp[1] > 1 && !can[1])) continue;
        const double len = ring_launch_tiles(rt, sp, p.heads, d.cus);
        if (len < best_len) {
          best_len = len;
          best[0] = sp[0];
          best[1] = sp[1];
        }
      }
      if (best_len > 0.95 * base) continue;  // within the estimate's error
      d.fr_split[r] = 1;
      for (int i = 0; i < 2; ++i) {
        const SegArgs& sa = d.fr_segs[size_t(r) * 2 + i];
        SegArgs& s0 = d.fr_split_segs[size_t(r) * 4 + i];
        SegArgs& s1 = d.fr_split_segs[size_t(r) * 4 + 2 + i];
        s0 = sa;
        s1 = sa;
        if (best[i] == 1) continue;
        s0.ksplit = s1.ksplit = 2;
        s0.tiles = s1.tiles = sa.tiles * 2;
        s0.diag = 0;
        s0.kv_full = s1.kv_full = int32_t(halves[i][0].back().end);
        s0.run0 = int32_t(all.size());
        all.insert(all.end(), halves[i][0].begin(), halves[i][0].end());
        s1.run0 = int32_t(all.size());
        all.insert(all.end(), halves[i][1].begin(), halves[i][1].end());
      }
    }
    if (!ok) return CP_ATTN_OK;  // served no more: the per-step launches take over
    // Two lanes pay off for short launches only: 8k/cp4/32 heads (at most
    // 128 key tiles per row tile) 0.62 against 0.71 ms per full forward;
    // 16k/cp4/16 heads (256) 1.14 against 1.13; 32k/cp8/32 heads (512) 8.56
    // against 7.65 (the two launches' waits and working sets collide)
    int64_t most = 0;
    for (const SegArgs& sa : d.fr_segs) most = std::max<int64_t>(most, sa.kv_full + (sa.diag ? sa.q_len : 0));
    d.fr_lanes = most <= 192 * 64;
    void* m = nullptr;
    CPA_HIP(hipMalloc(&m, all.size() * sizeof(RingRun)));
    d.fr_runs = static_cast<RingRun*>(m);
    CPA_HIP(hipMemcpy(d.fr_runs, all.data(), all.size() * sizeof(RingRun), hipMemcpyHostToDevice));
    CPA_HIP(hipMalloc(&m, size_t(p.cp) * sizeof(uint32_t)));
    d.fr_flags = static_cast<uint32_t*>(m);
    CPA_HIP(hipMemset(d.fr_flags, 0, size_t(p.cp) * sizeof(uint32_t)));
    CPA_HIP(hipMalloc(&m, size_t(p.cp) * sizeof(uint32_t)));
    d.fr_gflags = static_cast<uint32_t*>(m);
    CPA_HIP(hipMemset(d.fr_gflags, 0, size_t(p.cp) * sizeof(uint32_t)));
    CPA_HIP(hipDeviceSynchronize());  // zero before any stream of the plan reads them
    void* h = nullptr;
    CPA_HIP(hipHostMalloc(&h, sizeof(uint32_t), hipHostMallocCoherent | hipHostMallocMapped));
    d.fr_err = static_cast<uint32_t*>(h);
    *d.fr_err = 0;
    CPA_HIP(hipHostGetDevicePointer(&m, h, 0));
    d.fr_err_dev = static_cast<uint32_t*>(m);
    d.fr_ok = true;
  }
  if (!d.fr_ok) return CP_ATTN_OK;
  const int64_t need = 2 * align256(int64_t(p.cp - 1) * ws_layout(p).kv_bytes);
  if (d.fr_slots_bytes < need) {
    if (d.fr_slots) {  // earlier calls may still use it
      CPA_HIP(hipDeviceSynchronize());
      CPA_HIP(hipFree(d.fr_slots));
      d.fr_slots = nullptr;
      d.fr_slots_bytes = 0;
    }
    void* m = nullptr;
    if (hipMalloc(&m, size_t(need)) != hipSuccess) return fail(CP_ATTN_ENOWORKSPACE, "hipMalloc of the fused-ring slots failed");
    d.fr_slots = static_cast<char*>(m);
    d.fr_slots_bytes = need;
  }
  return CP_ATTN_OK;
}

// The second lane's streams, events, slots and flags (made once; the slots
// grow with the plan's need like the first lane's).
int ensure_fused_lane(Plan& p) {
  DeviceState& d = *p.dev;
  if (!d.fl_comp) {
    // (the compute stream last: it marks the lane as made, so a failure
    // part way leaves the rest to be made again by the next call)
    if (!d.fl_copy) CPA_HIP(hipStreamCreateWithFlags(&d.fl_copy, hipStreamNonBlocking));
    for (hipEvent_t* e : {&d.fl_enter, &d.fl_join, &d.fl_start, &d.fl_recv[0], &d.fl_recv[1]})
      if (!*e) CPA_HIP(hipEventCreateWithFlags(e, hipEventDisableTiming));
    if (!d.fl_flags) {
      void* m = nullptr;
      CPA_HIP(hipMalloc(&m, size_t(p.cp) * sizeof(uint32_t)));
      d.fl_flags = static_cast<uint32_t*>(m);
      CPA_HIP(hipMemset(d.fl_flags, 0, size_t(p.cp) * sizeof(uint32_t)));
      CPA_HIP(hipDeviceSynchronize());
    }
    CPA_HIP(hipStreamCreateWithFlags(&d.fl_comp, hipStreamNonBlocking));
  }
  bool odd_split = false;
  for (int r = 1; r < p.cp; r += 2) odd_split = odd_split || d.fr_split[size_t(r)];
  if (odd_split && !d.fl_split) {
    const WsLayout w = ws_layout(p);
    void* m = nullptr;
    const int64_t bytes = 2 * align256(w.o_bytes) + 2 * align256(w.lse_bytes) + align256(w.cnt_bytes);
    if (hipMalloc(&m, size_t(bytes)) != hipSuccess)
      return fail(CP_ATTN_ENOWORKSPACE, "hipMalloc of the second lane's key-split buffers failed");
    d.fl_split = static_cast<char*>(m);
  }
  if (d.fl_slots_bytes < d.fr_slots_bytes) {
    if (d.fl_slots) {
      CPA_HIP(hipDeviceSynchronize());
      CPA_HIP(hipFree(d.fl_slots));
      d.fl_slots = nullptr;
      d.fl_slots_bytes = 0;
    }
    void* m = nullptr;
    if (hipMalloc(&m, size_t(d.fr_slots_bytes)) != hipSuccess)
      return fail(CP_ATTN_ENOWORKSPACE, "hipMalloc of the second lane's fused-ring slots failed");
    d.fl_slots = static_cast<char*>(m);
    d.fl_slots_bytes = d.fr_slots_bytes;
  }
  return CP_ATTN_OK;
}

// lane 0: the caller's stream st, the copy stream and the first slots; lane
// 1 (odd ranks of a full forward): st is the second lane's compute stream,
// with its own copy stream, slots, flags and key-split buffers
int run_rank_fused(Plan& p, const RunCfg& c, const void* q, const void* k, const void* v, void* out, float* lse,
                   int r, hipStream_t st, int lane = 0) {
  DeviceState& d = *p.dev;
  const WsLayout w = ws_layout(p);
  const int P = p.cp;
  const bool l1 = lane == 1;
  hipStream_t const cps = l1 ? d.fl_copy : d.copy;
  char* const slots = l1 ? d.fl_slots : d.fr_slots;
  // graph capture: the epoch lives in flag word 0, advanced by a kernel
  // in every replay; otherwise the host numbers the call (never 0) and
  // passes the number by value to the signals and the launch
  const bool dev_epoch = c.capturing;
  uint32_t* const flags = dev_epoch ? d.fr_gflags : l1 ? d.fl_flags : d.fr_flags;
  hipEvent_t const ev_start = l1 ? d.fl_start : d.start;
  hipEvent_t const ev_recv[2] = {l1 ? d.fl_recv[0] : d.recv_done[0], l1 ? d.fl_recv[1] : d.recv_done[1]};
  uint32_t host_ep = 0;
  if (dev_epoch) {
    CPA_HIP(launch_ring_epoch(flags, st));
  } else {
    host_ep = ++d.fr_host_epoch;
    if (host_ep == 0) host_ep = d.fr_host_epoch = 1;
  }
  const int64_t kvs = w.kv_bytes;  // one slot of K (or V): the source's n_loc rows
  char* const k2 = slots;
  char* const v2 = slots + align256(int64_t(P - 1) * kvs);
  // the copy stream starts behind everything queued on st before this call
  // (an earlier call's kernel may still read the slots)
  CPA_HIP(hipEventRecord(ev_start, st));
  CPA_HIP(hipStreamWaitEvent(cps, ev_start, 0));
  for (int s = 1; s < P; ++s) {
    if (!d.fr_need[size_t(r) * P + s]) continue;  // no row of the rank sees that source (causal, contiguous)
    const RecvArgs ra = recv_ranges_to(p, k2 + int64_t(s - 1) * kvs, v2 + int64_t(s - 1) * kvs, k, v, p.step(r, s).src);
    // the first receive is needed soonest: the full grid; then the narrow one
    CPA_HIP(launch_recv(ra, s == 1 ? 0 : c.recv_blocks_fused, cps));
    if (dev_epoch) CPA_HIP(launch_ring_signal(flags + s, flags, cps));
    else CPA_HIP(launch_ring_signal_value(flags + s, host_ep, cps));
  }
  if (c.fused_ring == 3) {
    // staged: every receive done before the launch starts (no wait is polled)
    CPA_HIP(hipEventRecord(ev_recv[0], cps));
    CPA_HIP(hipStreamWaitEvent(st, ev_recv[0], 0));
  }
  StepArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.kv_bytes = p.seq_len * p.heads * p.head_dim * p.elem_bytes();
  a.k2 = k2;
  a.v2 = v2;
  a.kv2_bytes = int64_t(P - 1) * kvs;
  a.acc_o = reinterpret_cast<float*>(c.ws + w.acc_o);
  a.acc_lse = reinterpret_cast<float*>(c.ws + w.acc_lse);
  a.out = out;
  a.lse = lse;
  a.seq_len = p.seq_len;
  a.n_loc = int32_t(p.n_loc);
  a.kv_valid = int32_t(p.n_loc);
  a.heads = p.heads;
  a.scale = 1.0f / std::sqrt(float(p.head_dim));
  a.scale_log2 = a.scale * 1.4426950408889634f;
  a.out_f32 = 0;
  a.nseg = d.fr_nseg;
  const bool split = p.opt_ksplit && d.fr_split[size_t(r)];
  for (int i = 0; i < 2; ++i) {
    a.seg[i] = split ? d.fr_split_segs[size_t(r) * 4 + i] : d.fr_segs[size_t(r) * 2 + i];
    if (split) a.seg[2 + i] = d.fr_split_segs[size_t(r) * 4 + 2 + i];
    a.total_tiles += a.seg[i].tiles;
  }
  if (split && !l1) {
    for (int b = 0; b < 2; ++b) {
      a.split_o[b] = reinterpret_cast<float*>(c.ws + w.part_o[b]);
      a.split_lse[b] = reinterpret_cast<float*>(c.ws + w.part_lse[b]);
    }
    a.split_cnt = reinterpret_cast<int32_t*>(c.ws + w.split_cnt);
    // (the kernel leaves its counters at zero; a caller may have written the
    // workspace since: cleared by a kernel, which a graph may hold)
    CPA_HIP(launch_fill_words(c.ws + w.split_cnt, split_counters(p), 0u, st));
  } else if (split) {
    const int64_t ob = align256(w.o_bytes), lb = align256(w.lse_bytes);
    for (int b = 0; b < 2; ++b) {
      a.split_o[b] = reinterpret_cast<float*>(d.fl_split + b * ob);
      a.split_lse[b] = reinterpret_cast<float*>(d.fl_split + 2 * ob + b * lb);
    }
    a.split_cnt = reinterpret_cast<int32_t*>(d.fl_split + 2 * ob + 2 * lb);
    CPA_HIP(launch_fill_words(d.fl_split + 2 * ob + 2 * lb, split_counters(p), 0u, st));
  }
  a.runs = d.fr_runs;
  a.ring_flags = flags;
  a.ring_err = d.fr_err_dev;
  // test mode: an epoch no signal ever stores, and few polls
  a.ring_epoch_add = host_ep + (c.fused_ring == 2 ? 0x40000000u : 0u);
  a.ring_polls = c.fused_ring == 2 ? 16 : kRingPolls;
  // step timing: the one launch is reported under step 0
  const size_t ti = size_t(r) * P;
  if (c.timing) CPA_HIP(hipEventRecord(d.t0[ti], st));
  const hipError_t e = launch_attn_bf16_ring(a, st);
  if (e != hipSuccess) return fail(CP_ATTN_EHIP, std::string("fused ring launch: ") + hipGetErrorString(e));
  if (c.timing) {
    CPA_HIP(hipEventRecord(d.t1[ti], st));
    d.timed[ti] = 1;
  }
  if (c.capturing) {
    // a capture must join every stream it forked (the launch itself only
    // waits on the flags)
    CPA_HIP(hipEventRecord(ev_recv[1], cps));
    CPA_HIP(hipStreamWaitEvent(st, ev_recv[1], 0));
  }
  d.fr_last = split ? 2 : 1;
  return CP_ATTN_OK;
}

int run_rank(Plan& p, const RunCfg& c, const void* q, const void* k, const void* v, void* out, float* lse, int r,
             hipStream_t st) {
  DeviceState& d = *p.dev;
  const WsLayout w = ws_layout(p);
  char* ws = c.ws;
  const int P = p.cp;
  const bool serial = c.serial;
  const bool separate = p.opt_merge == 1;
  hipStream_t cs = serial ? st : d.copy;
  hipStream_t ms = serial ? st : d.merge;

  if (c.counters) {
    // this rank's work counters start at zero (a kernel: graph-safe)
    CPA_HIP(launch_fill_words(d.tile_cnt + size_t(r) * P, int64_t(P) * 2, 0u, st));
    for (int s = 0; s < P; ++s) d.counted[size_t(r) * P + s] = 1;
  }
  if (p.valid_rows(r) == 0) return CP_ATTN_OK;  // a rank of pad tokens only: nothing to compute or write
  if (fused_ring_served(p, c)) {
    CPA_TRY(ensure_fused_ring(p));
    if (p.dev->fr_ok) return run_rank_fused(p, c, q, k, v, out, lse, r, st);
  }
  p.dev->fr_last = 0;
  if (rank_splits(p, r)) {
    // The key split's per-tile counters: the kernels leave every counter they
    // use at zero, but nothing stops a caller from writing its workspace
    // between calls, so they are cleared (a kernel, so graph-safe) before any
    // step of a rank that splits.
    CPA_HIP(launch_fill_words(ws + w.split_cnt, split_counters(p), 0u, st));
  }
  // cross-stream events only where another stream waits on them: each
  // record/wait pair costs microseconds of queue latency per step
  bool any_side = false;
  for (int s = 0; s < P; ++s) any_side = any_side || side_recv(p, c, s);
  const bool copy_side = !serial && any_side;
  const bool merge_side = !serial && separate;
  if (copy_side || merge_side) {
    CPA_HIP(hipEventRecord(d.start, st));
    if (copy_side) CPA_HIP(hipStreamWaitEvent(cs, d.start, 0));
    if (merge_side) CPA_HIP(hipStreamWaitEvent(ms, d.start, 0));
  }
  const bool self_copy = kv_beyond_32bit(p);
  if (self_copy) CPA_HIP(launch_recv(recv_ranges(p, ws, k, v, r, 0), 0, st));  // own chunks into slot 0
  for (int s = 0; s < P; ++s) {
    const int b = s & 1;
    if (side_recv(p, c, s)) {
      // slot nb was last read by step s-1
      const int nb = (s + 1) & 1;
      if (!serial && s >= 1) CPA_HIP(hipStreamWaitEvent(cs, d.attn_done[nb], 0));
      CPA_TRY(recv_kv(p, c, k, v, p.step(r, s + 1).src, nb, serial || p.step(r, s).nseg == 0, cs));
      if (!serial) CPA_HIP(hipEventRecord(d.recv_done[nb], cs));
    }
    if (!serial && s >= 1 && side_recv(p, c, s - 1)) CPA_HIP(hipStreamWaitEvent(st, d.recv_done[b], 0));
    // part[b] is free once the merge of step s-2 has read it (step 0 writes
    // the running state directly and has no merge)
    if (separate && !serial && s >= 3) CPA_HIP(hipStreamWaitEvent(st, d.merge_done[b], 0));
    const size_t ti = size_t(r) * P + s;
    if (c.timing) CPA_HIP(hipEventRecord(d.t0[ti], st));
    CPA_TRY(launch_step(p, c, q, k, v, out, lse, r, s, b, st));
    if (c.timing) {
      CPA_HIP(hipEventRecord(d.t1[ti], st));
      d.timed[ti] = 1;
    }
    if (c.poison && (s >= 1 || self_copy)) {
      CPA_HIP(launch_poison(ws + w.slot_k[b], w.kv_bytes, st));
      CPA_HIP(launch_poison(ws + w.slot_v[b], w.kv_bytes, st));
    }
    // the copy stream's receive at step s+1 waits for this step; so does the
    // merge stream
    if ((!serial && side_recv(p, c, s + 1)) || merge_side) CPA_HIP(hipEventRecord(d.attn_done[b], st));
    if (separate && s > 0) {
      if (!serial) CPA_HIP(hipStreamWaitEvent(ms, d.attn_done[b], 0));
      CPA_TRY(launch_step_merge(p, ws, r, s, b, ms));
      if (c.poison) {
        CPA_HIP(launch_poison(ws + w.part_o[b], w.o_bytes, ms));
        CPA_HIP(launch_poison(ws + w.part_lse[b], w.lse_bytes, ms));
      }
      if (!serial) CPA_HIP(hipEventRecord(d.merge_done[b], ms));
    }
  }
  if (separate) {
    if (!serial) {
      CPA_HIP(hipEventRecord(d.merge_join, ms));
      CPA_HIP(hipStreamWaitEvent(st, d.merge_join, 0));
    }
    CPA_TRY(launch_rank_finalize(p, ws, out, lse, r, st));
  }
  return CP_ATTN_OK;
}

// ---- lockstep full forward ----
// Every rank's step s in one launch, as the ranks of a CP group run step s
// together: per step, the receives of all ranks on the copy stream, then one
// launch of the step kernel over every rank's tiles.  Each rank has its own
// receive slots and running state (a library-owned workspace); the document
// table stays the plan's.  Served for bf16 head_dim 128 with the fused merge
// and the side-stream receive (copy kernel or memcpy), without the serial,
// poison or step-timing modes and while step 0 reads K/V in place; otherwise
// the ranks run back to back.
bool lockstep_served(const Plan& p, const RunCfg& c) {
  return p.opt_lockstep && p.dtype == CP_ATTN_BF16 && p.head_dim == 128 && p.opt_merge == 0 &&
         (c.recv == 0 || c.recv == 1) && !c.serial && !c.poison && !c.timing && !kv_beyond_32bit(p) && p.cp > 1;
}

// bytes of one rank's slots and running state (the leading part of ws_layout)
int64_t lockstep_rank_bytes(const Plan& p) { return ws_layout(p).part_o[0]; }

int run_lockstep(Plan& p, const RunCfg& c0, const void* q, const void* k, const void* v, void* out, float* lse,
                 hipStream_t st) {
  DeviceState& d = *p.dev;
  d.fr_last = 0;
  const int P = p.cp;
  const int64_t rb = lockstep_rank_bytes(p);
  const int64_t tbl_bytes = int64_t(P) * P * int64_t(sizeof(StepArgs));
  const int64_t wgb_bytes = int64_t(P) * (P + 1) * 4;
  const int64_t need = rb * P + align256(tbl_bytes + wgb_bytes);
  if (d.ls_bytes < need) {
    if (d.ls_ws) {  // earlier calls may still use it
      CPA_HIP(hipDeviceSynchronize());
      CPA_HIP(hipFree(d.ls_ws));
      d.ls_ws = nullptr;
      d.ls_bytes = 0;
    }
    if (d.ls_host) {
      CPA_HIP(hipHostFree(d.ls_host));
      d.ls_host = nullptr;
    }
    if (hipMalloc(reinterpret_cast<void**>(&d.ls_ws), size_t(need)) != hipSuccess) {
      (void)hipGetLastError();
      d.ls_ws = nullptr;
      return fail(CP_ATTN_ENOWORKSPACE, "lockstep workspace allocation failed");
    }
    d.ls_bytes = need;
    CPA_HIP(hipHostMalloc(&d.ls_host, size_t(tbl_bytes + wgb_bytes), hipHostMallocDefault));
    if (!d.ls_uploaded) CPA_HIP(hipEventCreateWithFlags(&d.ls_uploaded, hipEventDisableTiming));
    d.ls_key.clear();
  }
  StepArgs* const tbl_dev = reinterpret_cast<StepArgs*>(d.ls_ws + rb * P);
  // the table and the ranges lie one after the other, as in the staging buffer
  int32_t* const wgb_dev = reinterpret_cast<int32_t*>(d.ls_ws + rb * P + tbl_bytes);
  auto rank_ws = [&](int r) { return d.ls_ws + rb * r; };
  // the table: every (rank, step)'s arguments and each step's workgroup ranges
  std::vector<int32_t> total(P, 0);
  const std::vector<intptr_t> key = {reinterpret_cast<intptr_t>(q), reinterpret_cast<intptr_t>(k),
                                     reinterpret_cast<intptr_t>(v), reinterpret_cast<intptr_t>(out),
                                     reinterpret_cast<intptr_t>(lse), intptr_t(c0.counters), intptr_t(p.doc_version),
                                     reinterpret_cast<intptr_t>(c0.ws)};
  {
    StepArgs* const tbl = static_cast<StepArgs*>(d.ls_host);
    int32_t* const wgb = reinterpret_cast<int32_t*>(static_cast<char*>(d.ls_host) + tbl_bytes);
    const bool fresh = d.ls_key == key;
    if (!fresh) CPA_HIP(hipEventSynchronize(d.ls_uploaded));  // the staging buffer's last upload has been read
    for (int s = 0; s < P; ++s) {
      int32_t* const w = wgb + int64_t(s) * (P + 1);
      w[0] = 0;
      for (int r = 0; r < P; ++r) {
        StepArgs& a = tbl[int64_t(s) * P + r];
        int32_t n = 0;
        if (p.step(r, s).nseg > 0 && p.valid_rows(r) > 0) {
          if (!fresh) a = make_step_args(p, c0, q, k, v, out, lse, r, s, s & 1, rank_ws(r), c0.ws, true);
          n = (a.total_tiles * a.heads + 7) / 8 * 8;
        } else if (!fresh) {
          a = StepArgs{};
        }
        w[r + 1] = w[r] + n;
      }
      total[s] = w[P];
    }
    if (!fresh) {
      CPA_HIP(hipMemcpyAsync(tbl_dev, d.ls_host, size_t(tbl_bytes + wgb_bytes), hipMemcpyHostToDevice, st));
      CPA_HIP(hipEventRecord(d.ls_uploaded, st));
      d.ls_key = key;
    }
  }
  if (c0.counters) {
    CPA_HIP(launch_fill_words(d.tile_cnt, int64_t(P) * P * 2, 0u, st));
    for (int i = 0; i < P * P; ++i) d.counted[size_t(i)] = 1;
  }
  hipStream_t cs = d.copy;
  CPA_HIP(hipEventRecord(d.start, st));
  CPA_HIP(hipStreamWaitEvent(cs, d.start, 0));
  for (int s = 0; s < P; ++s) {
    const int b = s & 1;
    if (s + 1 < P) {
      // every rank's receive of step s + 1 into its slot nb, last read by step s - 1
      const int nb = (s + 1) & 1;
      if (s >= 1) CPA_HIP(hipStreamWaitEvent(cs, d.attn_done[nb], 0));
      for (int r = 0; r < P; ++r) {
        if (p.valid_rows(r) == 0) continue;
        RunCfg cr = c0;
        cr.ws = rank_ws(r);
        CPA_TRY(recv_kv(p, cr, k, v, p.step(r, s + 1).src, nb, false, cs));
      }
      CPA_HIP(hipEventRecord(d.recv_done[nb], cs));
    }
    if (s >= 1) CPA_HIP(hipStreamWaitEvent(st, d.recv_done[b], 0));
    const hipError_t e = launch_attn_bf16_ranks(tbl_dev + int64_t(s) * P, wgb_dev + int64_t(s) * (P + 1), P, total[s],
                                                !p.doc_starts.empty(), st);
    if (e != hipSuccess) return fail(CP_ATTN_EHIP, std::string("lockstep attention launch: ") + hipGetErrorString(e));
    if (s + 2 < P) CPA_HIP(hipEventRecord(d.attn_done[b], st));
  }
  return CP_ATTN_OK;
}

int check_plan(cp_attn_plan_t h) {
  if (!h || !h->p) return fail(CP_ATTN_EINVAL, "plan is null");
  return CP_ATTN_OK;
}

// lse_align: the alignment demanded of lse (it is only ever written with
// 4-byte stores; entry points that document 4 pass 4)
int check_io(const void* q, const void* k, const void* v, const void* out, const void* lse, int lse_align = 16) {
  const void* ptrs[5] = {q, k, v, out, lse};
  const char* names[5] = {"q", "k", "v", "out", "lse"};
  for (int i = 0; i < 5; ++i) {
    if (!ptrs[i]) return fail(CP_ATTN_EINVAL, std::string(names[i]) + " is null");
    const uintptr_t al = i == 4 ? uintptr_t(lse_align) : 16u;
    if (reinterpret_cast<uintptr_t>(ptrs[i]) % al != 0)
      return fail(CP_ATTN_EINVAL, std::string(names[i]) + " is not " + std::to_string(al) + "-byte aligned");
  }
  return CP_ATTN_OK;
}

void reset_timing(Plan& p) {
  DeviceState& d = *p.dev;
  d.timed.assign(size_t(p.cp) * p.cp, 0);
  d.counted.assign(size_t(p.cp) * p.cp, 0);
}

// ---- the no-allocation forward ----
// The workspace of cp_attn_rank_forward_noalloc: a file-scope device array.
// Each GPU the library runs on holds its own copy, at its own address, until
// the process ends.  On the host, `scratch` names a host-side stand-in, not
// device memory: host code uses only the address hipGetSymbolAddress returns
// for the current device (scratch_base), never the array's name.
constexpr int64_t kScratchBytes = CP_ATTN_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Device address of `scratch` on device `dev` (the current device), looked up
// once per device and kept.
int scratch_base(int dev, char** out) {
  static std::mutex mu;
  static void* base[kMaxDevices] = {};
  if (dev < 0 || dev >= kMaxDevices) return fail(CP_ATTN_EUNSUPPORTED, "device index beyond the scratch table");
  std::lock_guard<std::mutex> lock(mu);
  if (!base[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(CP_ATTN_EHIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    base[dev] = ptr;
  }
  *out = static_cast<char*>(base[dev]);
  return CP_ATTN_OK;
}

void drop_graph(DeviceState& d) {
  if (d.graph) (void)hipGraphExecDestroy(d.graph);
  d.graph = nullptr;
  d.graph_key.clear();
}

// Graph mode: the forward of one rank (rank >= 0) or of every rank (-1) is
// recorded once, by stream capture on the library's capture stream (the copy
// and merge streams join through their events), and the executable graph is
// replayed on the caller's stream while the buffers, the workspace, the side
// streams and the options are the ones it was recorded with; anything else
// records it again.  Replays read the buffers' current contents.
int run_graph(Plan& p, const void* q, const void* k, const void* v, void* out, float* lse, int rank,
              hipStream_t st) {
  DeviceState& d = *p.dev;
  const std::vector<intptr_t> key = {
      intptr_t(q), intptr_t(k), intptr_t(v), intptr_t(out), intptr_t(lse), rank,
      intptr_t(d.ws), intptr_t(d.copy), intptr_t(d.merge), p.dtype, p.opt_merge, p.opt_serialize,
      p.opt_recv, p.opt_poison, p.opt_recv_blocks, p.opt_ksplit, p.opt_counters, intptr_t(p.doc_version),
      p.opt_fused_ring};
  if (!d.graph || key != d.graph_key) {
    drop_graph(d);
    // the fused ring's buffers and table are made outside the capture
    if (fused_ring_served(p, plan_cfg(p, true))) CPA_TRY(ensure_fused_ring(p));
    if (!d.capture) CPA_HIP(hipStreamCreateWithFlags(&d.capture, hipStreamNonBlocking));
    CPA_HIP(hipStreamBeginCapture(d.capture, hipStreamCaptureModeThreadLocal));
    int rc = CP_ATTN_OK;
    for (int r = rank < 0 ? 0 : rank; r < (rank < 0 ? p.cp : rank + 1) && rc == CP_ATTN_OK; ++r)
      rc = run_rank(p, plan_cfg(p, true), q, k, v, out, lse, r, d.capture);
    hipGraph_t g = nullptr;
    const hipError_t ec = hipStreamEndCapture(d.capture, &g);
    if (rc != CP_ATTN_OK) {
      if (g) (void)hipGraphDestroy(g);
      return rc;
    }
    if (ec != hipSuccess) return fail(CP_ATTN_EHIP, std::string("hipStreamEndCapture: ") + hipGetErrorString(ec));
    const hipError_t ei = hipGraphInstantiate(&d.graph, g, nullptr, nullptr, 0);
    (void)hipGraphDestroy(g);
    if (ei != hipSuccess) {
      d.graph = nullptr;
      return fail(CP_ATTN_EHIP, std::string("hipGraphInstantiate: ") + hipGetErrorString(ei));
    }
    d.graph_key = key;
  }
  CPA_HIP(hipGraphLaunch(d.graph, st));
  if (p.opt_counters)  // the graph zeroes and fills the counters of the ranks it holds
    for (int r = rank < 0 ? 0 : rank; r < (rank < 0 ? p.cp : rank + 1); ++r)
      for (int s = 0; s < p.cp; ++s) d.counted[size_t(r) * p.cp + s] = 1;
  return CP_ATTN_OK;
}

// ---- backward ----

// Rows and keys per workgroup of the backward kernels the plan uses.
void bwd_tile_sizes(const Plan& p, int* rows, int* keys) {
  if (bwd_mfma(p.dtype == CP_ATTN_BF16, p.head_dim)) {
    *rows = bwd_mfma_rows();
    *keys = bwd_mfma_keys();
  } else {
    *rows = bwd_generic_tile();
    *keys = bwd_generic_tile();
  }
}

// The backward over the natural-order K/V as one source: local row runs of
// rank r (its chunks) whose key prefix is every key before the chunk
// (causal, the chunk's own keys as the diagonal) or every key (bidirectional),
// the run that sees more keys first.  The keys of all ring steps of a row are
// then one prefix of the natural order, so one launch of each kernel covers
// every step: the keys each step's source holds, in natural order instead of
// step order.  Served for the matrix-core kernels without documents or
// padding while a K/V row offset stays below 2^31 bytes.
bool bwd_fused_served(const Plan& p) {
  if (!p.opt_bwd_fused || !bwd_mfma(p.dtype == CP_ATTN_BF16, p.head_dim)) return false;
  if (!p.doc_starts.empty() || p.padded_len != p.seq_len) return false;
  return p.seq_len * int64_t(p.heads) * p.head_dim * p.elem_bytes() < (int64_t(1) << 31);
}

void bwd_fused_args(const Plan& p, int r, int bt_rows, int bt_keys, BwdArgs& a) {
  const int64_t C = p.layout == 1 ? p.chunk : p.n_loc;
  const int nch = p.layout == 1 ? 2 : 1;
  Segment segs[2];
  for (int c = 0; c < nch; ++c) {
    Segment& g = segs[c];
    g.q_start = c * C;
    g.q_len = C;
    g.q_global = p.global_row(r, c * C);
    g.kv_full = p.causal ? g.q_global : p.seq_len;
    g.diag = p.causal ? 1 : 0;
  }
  if (nch == 2 && segs[1].kv_full > segs[0].kv_full) std::swap(segs[0], segs[1]);
  a.kv_lo = 0;
  a.kv_hi = 0;
  a.kv_split = int32_t(p.seq_len);
  a.kv_valid = int32_t(p.seq_len);
  a.nseg = nch;
  a.total_tiles = 0;
  a.seg[1] = SegArgs{};
  int64_t maxpre = 0;
  for (int i = 0; i < nch; ++i) {
    const Segment& g = segs[i];
    SegArgs& x = a.seg[i];
    x = SegArgs{};
    x.q_global = g.q_global;
    x.q_start = int32_t(g.q_start);
    x.q_len = int32_t(g.q_len);
    x.kv_full = int32_t(g.kv_full);
    x.diag = g.diag;
    x.epi = 1;  // dQ written once
    x.ksplit = 1;
    x.tiles = int32_t((g.q_len + bt_rows - 1) / bt_rows);
    a.total_tiles += x.tiles;
    maxpre = std::max<int64_t>(maxpre, g.kv_full + (g.diag ? g.q_len : 0));
  }
  a.key_tiles = int32_t((maxpre + bt_keys - 1) / bt_keys);
  a.doc = nullptr;
}

// Rank r's share of the backward on one stream: D_i of its rows, then per
// ring step the key-major (dK, dV) and row-major (dQ) kernels of the step's
// segments (CP_ATTN_OPT_BWD_FUSED 1: dQ of every step in one launch; 2:
// dK, dV of every step in one launch too).  K and V are read in place at the source's natural rows, and the
// source's dK, dV are accumulated there: on a real ring those partial sums
// travel with the K/V chunks and arrive home complete after cp steps.
int run_rank_backward(Plan& p, const void* q, const void* k, const void* v, const void* out, const float* lse,
                      const void* dout, float* dq, float* dk, float* dv, int r, hipStream_t st) {
  if (p.valid_rows(r) == 0) return CP_ATTN_OK;  // a rank of pad tokens only
  DeviceState& d = *p.dev;
  const WsLayout w = ws_layout(p);
  char* ws = static_cast<char*>(d.ws);
  const bool bf16 = p.dtype == CP_ATTN_BF16;
  int bt_rows = 0, bt_keys = 0;
  bwd_tile_sizes(p, &bt_rows, &bt_keys);
  BwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.dout = dout;
  a.lse = lse;
  a.delta = reinterpret_cast<float*>(ws + w.acc_lse);  // the forward's running-LSE region, [H][n_loc]
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.seq_len = p.seq_len;
  a.n_loc = int32_t(p.n_loc);
  a.heads = p.heads;
  a.scale = 1.0f / std::sqrt(float(p.head_dim));
  a.scale_log2 = a.scale * 1.4426950408889634f;
  const int64_t split = p.layout == 1 ? p.chunk : p.n_loc;
  a.delta_rows = p.valid_rows(r);
  a.delta_lo = p.chunk_of(r, 0) * p.chunk;
  a.delta_hi = p.layout == 1 ? p.chunk_of(r, 1) * p.chunk : 0;
  a.delta_split = split;
  CPA_HIP(launch_bwd_delta(a, bf16, p.head_dim, st));
  const bool fused = bwd_fused_served(p);
  // (the one dQ launch of mode 1 on a side stream beside the per-step dK/dV
  // launches measured slower than in turn: 3.99 against 3.82 ms at 32k/cp8)
  if (fused) {
    BwdArgs f = a;
    bwd_fused_args(p, r, bt_rows, bt_keys, f);
    if (p.opt_bwd_fused == 1) f.key_tiles = 0;  // dK, dV per step below
    const hipError_t e = launch_bwd_bf16_d128(f, p.opt_bwd_keys == 0, st);
    if (e != hipSuccess) return fail(CP_ATTN_EHIP, std::string("backward launch: ") + hipGetErrorString(e));
    if (p.opt_bwd_fused == 2) return CP_ATTN_OK;
  }
  for (int s = 0; s < p.cp; ++s) {
    const StepDesc& sd = p.step(r, s);
    if (sd.nseg == 0) continue;
    const int j = sd.src;
    a.kv_lo = int32_t(p.chunk_of(j, 0) * p.chunk);
    a.kv_hi = p.layout == 1 ? int32_t(p.chunk_of(j, 1) * p.chunk) : 0;
    a.kv_split = int32_t(split);
    a.kv_valid = int32_t(p.valid_rows(j));
    a.nseg = sd.nseg;
    a.total_tiles = 0;
    a.seg[1] = SegArgs{};
    int64_t maxpre = 0;  // longest key prefix of the step's rows
    for (int i = 0; i < sd.nseg; ++i) {
      const Segment& g = sd.seg[i];
      SegArgs& x = a.seg[i];
      x.q_global = g.q_global;
      x.q_start = int32_t(g.q_start);
      x.q_len = int32_t(g.q_len);
      x.kv_full = int32_t(g.kv_full);
      x.diag = g.diag;
      x.epi = g.first;
      x.ksplit = 1;
      x.tiles = int32_t((g.q_len + bt_rows - 1) / bt_rows);
      a.total_tiles += x.tiles;
      maxpre = std::max<int64_t>(maxpre, g.kv_full + (g.diag ? g.q_len : 0));
    }
    a.key_tiles = int32_t((maxpre + bt_keys - 1) / bt_keys);
    if (fused) a.total_tiles = 0;  // dQ done above
    set_doc(p, ws, a, j);
    const hipError_t e = bwd_mfma(bf16, p.head_dim) ? launch_bwd_bf16_d128(a, p.opt_bwd_keys == 0, st)
                                                    : launch_bwd_generic(a, bf16, p.head_dim, st);
    if (e != hipSuccess) return fail(CP_ATTN_EHIP, std::string("backward launch: ") + hipGetErrorString(e));
  }
  return CP_ATTN_OK;
}

int check_bwd_io(const void* dout, const void* dq, const void* dk, const void* dv) {
  const void* ptrs[4] = {dout, dq, dk, dv};
  const char* names[4] = {"dout", "dq", "dk", "dv"};
  for (int i = 0; i < 4; ++i) {
    if (!ptrs[i]) return fail(CP_ATTN_EINVAL, std::string(names[i]) + " is null");
    if (!aligned16(ptrs[i])) return fail(CP_ATTN_EINVAL, std::string(names[i]) + " is not 16-byte aligned");
  }
  return CP_ATTN_OK;
}

}  // namespace
}  // namespace cpattn

using namespace cpattn;

#define CPA_GUARD_BEGIN try {
#define CPA_GUARD_END                                              \
  }                                                                \
  catch (const std::bad_alloc&) {                                  \
    return fail(CP_ATTN_EINVAL, "host allocation failed");         \
  }                                                                \
  catch (...) {                                                    \
    return fail(CP_ATTN_EINVAL, "unexpected C++ exception");       \
  }

extern "C" {

int cp_attn_plan(int64_t seq_len, int cp_size, int heads, int head_dim, int causal, int layout,
                 cp_attn_plan_t* out) {
  CPA_GUARD_BEGIN
  if (!out) return fail(CP_ATTN_EINVAL, "out is null");
  *out = nullptr;
  Plan* p = nullptr;
  std::string err;
  const int rc = make_plan(seq_len, cp_size, heads, head_dim, causal, layout, &p, &err);
  if (rc != CP_ATTN_OK) return fail(rc, err);
  p->dev = new DeviceState;
  *out = new cp_attn_plan_s{p};
  return CP_ATTN_OK;
  CPA_GUARD_END
}

int cp_attn_plan_destroy(cp_attn_plan_t h) {
  CPA_GUARD_BEGIN
  if (!h) return CP_ATTN_OK;
  Plan* p = h->p;
  int rc = CP_ATTN_OK;
  if (p && p->dev) {
    DeviceState& d = *p->dev;
    if (d.device >= 0) {
      int cur = 0;
      (void)hipGetDevice(&cur);
      (void)hipSetDevice(d.device);
      if (hipDeviceSynchronize() != hipSuccess) rc = fail(CP_ATTN_EHIP, "hipDeviceSynchronize failed in destroy");
      drop_graph(d);
      if (d.capture) (void)hipStreamDestroy(d.capture);
      if (d.tile_cnt) (void)hipFree(d.tile_cnt);
      if (d.ls_ws) (void)hipFree(d.ls_ws);
      if (d.ls_host) (void)hipHostFree(d.ls_host);
      if (d.ls_uploaded) (void)hipEventDestroy(d.ls_uploaded);
      if (d.fr_slots) (void)hipFree(d.fr_slots);
      if (d.fr_flags) (void)hipFree(d.fr_flags);
      if (d.fr_gflags) (void)hipFree(d.fr_gflags);
      if (d.fr_runs) (void)hipFree(d.fr_runs);
      if (d.fr_err) (void)hipHostFree(d.fr_err);
      if (d.fl_slots) (void)hipFree(d.fl_slots);
      if (d.fl_flags) (void)hipFree(d.fl_flags);
      if (d.fl_split) (void)hipFree(d.fl_split);
      if (d.fl_comp) (void)hipStreamDestroy(d.fl_comp);
      if (d.fl_copy) (void)hipStreamDestroy(d.fl_copy);
      for (hipEvent_t e : {d.fl_enter, d.fl_join, d.fl_start, d.fl_recv[0], d.fl_recv[1]})
        if (e) (void)hipEventDestroy(e);
      if (d.own_ws && d.ws) (void)hipFree(d.ws);
      if (d.own_copy && d.copy) (void)hipStreamDestroy(d.copy);
      if (d.own_merge && d.merge) (void)hipStreamDestroy(d.merge);
      if (d.events_ready) {
        (void)hipEventDestroy(d.start);
        (void)hipEventDestroy(d.merge_join);
        for (int b = 0; b < 2; ++b) {
          (void)hipEventDestroy(d.recv_done[b]);
          (void)hipEventDestroy(d.attn_done[b]);
          (void)hipEventDestroy(d.merge_done[b]);
        }
      }
      for (hipEvent_t e : d.t0) (void)hipEventDestroy(e);
      for (hipEvent_t e : d.t1) (void)hipEventDestroy(e);
      (void)hipSetDevice(cur);
    }
    delete p->dev;
  }
  delete p;
  delete h;
  return rc;
  CPA_GUARD_END
}

int cp_attn_set_dtype(cp_attn_plan_t h, int dtype) {
  CPA_TRY(check_plan(h));
  if (dtype != CP_ATTN_BF16 && dtype != CP_ATTN_FP32) return fail(CP_ATTN_EINVAL, "dtype must be BF16 or FP32");
  h->p->dtype = dtype;
  return CP_ATTN_OK;
}

int cp_attn_set_option(cp_attn_plan_t h, int option, int value) {
  CPA_TRY(check_plan(h));
  Plan& p = *h->p;
  switch (option) {
    case CP_ATTN_OPT_MERGE:
      if (value != 0 && value != 1) return fail(CP_ATTN_EINVAL, "merge option must be 0 or 1");
      p.opt_merge = value;
      return CP_ATTN_OK;
    case CP_ATTN_OPT_SERIALIZE:
      p.opt_serialize = value != 0;
      return CP_ATTN_OK;
    case CP_ATTN_OPT_RECV:
      if (value < 0 || value > 3) return fail(CP_ATTN_EINVAL, "recv option must be 0, 1, 2 or 3");
      p.opt_recv = value;
      return CP_ATTN_OK;
    case CP_ATTN_OPT_POISON:
      p.opt_poison = value != 0;
      return CP_ATTN_OK;
    case CP_ATTN_OPT_STEP_TIMING:
      p.opt_step_timing = value != 0;
      return CP_ATTN_OK;
    case CP_ATTN_OPT_RECV_BLOCKS:
      if (value < -1) return fail(CP_ATTN_EINVAL, "recv_blocks must be >= -1");
      p.opt_recv_blocks = value;
      return CP_ATTN_OK;
    case CP_ATTN_OPT_GRAPH:
      if (value != 0 && value != 1) return fail(CP_ATTN_EINVAL, "graph option must be 0 or 1");
      p.opt_graph = value;
      return CP_ATTN_OK;
    case CP_ATTN_OPT_KSPLIT:
      if (value != 0 && value != 1) return fail(CP_ATTN_EINVAL, "ksplit option must be 0 or 1");
      p.opt_ksplit = value;
      return CP_ATTN_OK;
    case CP_ATTN_OPT_BWD_KEYS:
      if (value != 0 && value != 1) return fail(CP_ATTN_EINVAL, "CP_ATTN_OPT_BWD_KEYS must be 0 or 1");
      p.opt_bwd_keys = value;
      return CP_ATTN_OK;
    case CP_ATTN_OPT_LOCKSTEP:
      if (value != 0 && value != 1) return fail(CP_ATTN_EINVAL, "CP_ATTN_OPT_LOCKSTEP must be 0 or 1");
      p.opt_lockstep = value;
      return CP_ATTN_OK;
    case CP_ATTN_OPT_FUSED_RING:
      if (value < 0 || value > 3) return fail(CP_ATTN_EINVAL, "CP_ATTN_OPT_FUSED_RING must be 0, 1, 2 or 3");
      p.opt_fused_ring = value;
      return CP_ATTN_OK;
    case CP_ATTN_OPT_BWD_FUSED:
      if (value < 0 || value > 2) return fail(CP_ATTN_EINVAL, "CP_ATTN_OPT_BWD_FUSED must be 0, 1 or 2");
      p.opt_bwd_fused = value;
      return CP_ATTN_OK;
    case CP_ATTN_OPT_COUNTERS:
      if (value != 0 && value != 1) return fail(CP_ATTN_EINVAL, "counters option must be 0 or 1");
      p.opt_counters = value;
      return CP_ATTN_OK;
    default:
      return fail(CP_ATTN_EINVAL, "unknown option");
  }
}

int cp_attn_fused_ring_active(cp_attn_plan_t h, int32_t* active) {
  CPA_TRY(check_plan(h));
  if (!active) return fail(CP_ATTN_EINVAL, "active is null");
  *active = h->p->dev->fr_last;
  return CP_ATTN_OK;
}

int cp_attn_ring_wait_timeouts(cp_attn_plan_t h, int32_t* timed_out) {
  CPA_TRY(check_plan(h));
  if (!timed_out) return fail(CP_ATTN_EINVAL, "timed_out is null");
  DeviceState& d = *h->p->dev;
  *timed_out = d.fr_err ? int32_t(__atomic_exchange_n(d.fr_err, 0u, __ATOMIC_SEQ_CST) != 0) : 0;
  return CP_ATTN_OK;
}

int cp_attn_workspace_bytes(cp_attn_plan_t h, int64_t* bytes) {
  CPA_TRY(check_plan(h));
  if (!bytes) return fail(CP_ATTN_EINVAL, "bytes is null");
  *bytes = ws_layout(*h->p).total;
  return CP_ATTN_OK;
}

int cp_attn_set_workspace(cp_attn_plan_t h, void* ptr, int64_t bytes) {
  CPA_TRY(check_plan(h));
  DeviceState& d = *h->p->dev;
  if (ptr && (reinterpret_cast<uintptr_t>(ptr) & 255u)) return fail(CP_ATTN_EINVAL, "workspace not 256-byte aligned");
  if (ptr && bytes < ws_layout(*h->p).total) return fail(CP_ATTN_ENOWORKSPACE, "workspace too small");
  if (d.own_ws && d.ws) {
    CPA_HIP(hipDeviceSynchronize());
    CPA_HIP(hipFree(d.ws));
  }
  d.ws = ptr;
  d.ws_bytes = ptr ? bytes : 0;
  d.own_ws = false;
  d.doc_uploaded = -1;
  return CP_ATTN_OK;
}

int cp_attn_set_documents(cp_attn_plan_t h, const int64_t* starts, int64_t count) {
  CPA_GUARD_BEGIN
  CPA_TRY(check_plan(h));
  Plan& p = *h->p;
  std::string err;
  const int rc = set_documents(p, starts, count, &err);
  if (rc != CP_ATTN_OK) return fail(rc, err);
  drop_graph(*p.dev);
  return CP_ATTN_OK;
  CPA_GUARD_END
}

int cp_attn_set_streams(cp_attn_plan_t h, void* copy_stream, void* merge_stream) {
  CPA_TRY(check_plan(h));
  DeviceState& d = *h->p->dev;
  if (d.own_copy && d.copy) CPA_HIP(hipStreamDestroy(d.copy));
  if (d.own_merge && d.merge) CPA_HIP(hipStreamDestroy(d.merge));
  d.copy = static_cast<hipStream_t>(copy_stream);
  d.merge = static_cast<hipStream_t>(merge_stream);
  d.own_copy = d.own_merge = false;
  return CP_ATTN_OK;
}

int cp_attn_rank_forward(cp_attn_plan_t h, const void* q, const void* k, const void* v, void* out, float* lse,
                         int rank, void* stream) {
  CPA_GUARD_BEGIN
  CPA_TRY(check_plan(h));
  Plan& p = *h->p;
  if (rank < 0 || rank >= p.cp) return fail(CP_ATTN_EINVAL, "rank outside [0, cp_size)");
  CPA_TRY(check_io(q, k, v, out, lse));
  CPA_TRY(ensure_device(p));
  reset_timing(p);
  // (a rank of pad tokens only has nothing to record)
  if (p.opt_graph && p.valid_rows(rank) > 0) return run_graph(p, q, k, v, out, lse, rank, static_cast<hipStream_t>(stream));
  return run_rank(p, plan_cfg(p, false), q, k, v, out, lse, rank, static_cast<hipStream_t>(stream));
  CPA_GUARD_END
}

// All-gather variant: rank r's rows against the whole natural-order K/V in one
// launch of the step kernel.  Each owned chunk is one segment whose keys are
// the global prefix before the chunk (every row sees it) plus the causal
// diagonal inside the chunk (all keys when bidirectional); the key map is the
// identity, and the epilogue writes O and LSE straight to the global rows.
int cp_attn_allgather_forward(cp_attn_plan_t h, const void* q, const void* k, const void* v, void* out, float* lse,
                              int rank, void* stream) {
  CPA_GUARD_BEGIN
  CPA_TRY(check_plan(h));
  Plan& p = *h->p;
  if (rank < 0 || rank >= p.cp) return fail(CP_ATTN_EINVAL, "rank outside [0, cp_size)");
  CPA_TRY(check_io(q, k, v, out, lse));
  CPA_TRY(ensure_device(p, !p.doc_starts.empty()));
  const bool bf16 = p.dtype == CP_ATTN_BF16;
  const int bm = bf16 ? attn_bf16_block_m(p.head_dim) : attn_f32_block_m();
  if (p.seq_len * p.heads * p.head_dim * p.elem_bytes() > int64_t(UINT32_MAX))
    return fail(CP_ATTN_EUNSUPPORTED, "K/V beyond 4 GiB: too large for the all-gather launch");
  StepArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.kv_bytes = p.seq_len * p.heads * p.head_dim * p.elem_bytes();
  a.kv_lo = 0;
  a.kv_hi = 0;
  a.kv_split = int32_t(p.seq_len);
  a.out = out;
  a.lse = lse;
  a.seq_len = p.seq_len;
  a.n_loc = int32_t(p.seq_len);  // keys addressable through the identity map
  a.kv_valid = int32_t(p.seq_len);
  a.heads = p.heads;
  a.scale = 1.0f / std::sqrt(float(p.head_dim));
  a.scale_log2 = a.scale * 1.4426950408889634f;
  a.out_f32 = p.dtype == CP_ATTN_FP32;
  const int nch = p.layout == 1 ? 2 : 1;
  for (int c = 0; c < nch; ++c) {  // real rows of each owned chunk
    const int64_t len = p.valid_in_chunk(p.chunk_of(rank, c));
    if (len == 0) continue;
    const int64_t g0 = p.global_row(rank, c * p.chunk);
    SegArgs& x = a.seg[a.nseg++];
    x.q_global = g0;
    x.q_start = int32_t(c * p.chunk);
    x.q_len = int32_t(len);
    x.kv_full = int32_t(p.causal ? g0 : p.seq_len);
    x.diag = p.causal ? 1 : 0;
    x.ksplit = 1;
    x.tiles = int32_t((len + bm - 1) / bm);
    x.epi = kEpiInit | kEpiFinal;
    a.total_tiles += x.tiles;
  }
  if (a.nseg == 0) return CP_ATTN_OK;  // a rank of pad only
  set_doc(p, static_cast<const char*>(p.dev->ws), a, -1);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const hipError_t e = bf16 ? launch_attn_bf16(a, p.head_dim, st) : launch_attn_f32(a, p.head_dim, st);
  if (e != hipSuccess) return fail(CP_ATTN_EHIP, std::string("attention launch: ") + hipGetErrorString(e));
  return CP_ATTN_OK;
  CPA_GUARD_END
}

// Ulysses: the all-to-all of every rank at once, and one rank's attention over
// every token of its head slice (one launch of the step kernel, identity key
// map, the whole sequence as one segment).
int cp_attn_ulysses_a2a(cp_attn_plan_t h, const void* src, void* dst, int to_heads, void* stream) {
  CPA_GUARD_BEGIN
  CPA_TRY(check_plan(h));
  Plan& p = *h->p;
  if (p.heads % p.cp != 0) return fail(CP_ATTN_EUNSUPPORTED, "Ulysses needs heads divisible by cp_size");
  if (!src || !dst) return fail(CP_ATTN_EINVAL, "src or dst is null");
  if (!aligned16(src) || !aligned16(dst)) return fail(CP_ATTN_EINVAL, "src or dst not 16-byte aligned");
  if (to_heads != 0 && to_heads != 1) return fail(CP_ATTN_EINVAL, "to_heads must be 0 or 1");
  CPA_TRY(ensure_device(p, false));
  UlyssesArgs u{};
  u.src = src;
  u.dst = dst;
  u.to_heads = to_heads;
  u.cp = p.cp;
  u.zigzag = p.layout == 1;
  u.seq_len = p.seq_len;
  u.chunk = p.chunk;
  u.n_loc = p.n_loc;
  u.heads = p.heads;
  u.head_vec = int64_t(p.head_dim) * p.elem_bytes() / 16;
  CPA_HIP(launch_ulysses(u, static_cast<hipStream_t>(stream)));
  return CP_ATTN_OK;
  CPA_GUARD_END
}

int cp_attn_ulysses_forward(cp_attn_plan_t h, const void* q, const void* k, const void* v, void* out, float* lse,
                            void* stream) {
  CPA_GUARD_BEGIN
  CPA_TRY(check_plan(h));
  Plan& p = *h->p;
  if (p.heads % p.cp != 0) return fail(CP_ATTN_EUNSUPPORTED, "Ulysses needs heads divisible by cp_size");
  CPA_TRY(check_io(q, k, v, out, lse, 4));  // lse may be a row slice of a [heads][S] array
  const int32_t group = p.heads / p.cp;
  if (p.seq_len * group * p.head_dim * p.elem_bytes() > int64_t(UINT32_MAX))
    return fail(CP_ATTN_EUNSUPPORTED, "a head slice beyond 4 GiB");
  CPA_TRY(ensure_device(p, !p.doc_starts.empty()));
  const bool bf16 = p.dtype == CP_ATTN_BF16;
  const int bm = bf16 ? attn_bf16_block_m(p.head_dim) : attn_f32_block_m();
  StepArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.kv_bytes = p.seq_len * group * p.head_dim * p.elem_bytes();
  a.kv_lo = 0;
  a.kv_hi = 0;
  a.kv_split = int32_t(p.seq_len);
  a.out = out;
  a.lse = lse;
  a.seq_len = p.seq_len;
  a.n_loc = int32_t(p.seq_len);
  a.kv_valid = int32_t(p.seq_len);
  a.heads = group;
  a.scale = 1.0f / std::sqrt(float(p.head_dim));
  a.scale_log2 = a.scale * 1.4426950408889634f;
  a.out_f32 = p.dtype == CP_ATTN_FP32;
  a.nseg = 1;
  SegArgs& x = a.seg[0];
  x.q_global = 0;
  x.q_start = 0;
  x.q_len = int32_t(p.seq_len);
  x.kv_full = p.causal ? 0 : int32_t(p.seq_len);
  x.diag = p.causal ? 1 : 0;
  x.ksplit = 1;
  x.tiles = int32_t((p.seq_len + bm - 1) / bm);
  x.epi = kEpiInit | kEpiFinal;
  a.total_tiles = x.tiles;
  set_doc(p, static_cast<const char*>(p.dev->ws), a, -1);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const hipError_t e = bf16 ? launch_attn_bf16(a, p.head_dim, st) : launch_attn_f32(a, p.head_dim, st);
  if (e != hipSuccess) return fail(CP_ATTN_EHIP, std::string("attention launch: ") + hipGetErrorString(e));
  return CP_ATTN_OK;
  CPA_GUARD_END
}

// The same steps as cp_attn_rank_forward on the static scratch, without any
// allocation: no plan workspace, no side streams or events (every kernel on
// the caller's stream, the ring receive inside the step kernels where they
// support it, else a full-grid copy kernel before the step), no step timing
// or work counters.  The key-split counters are cleared by run_rank's fill
// kernel; every other scratch region is written before it is read.
int cp_attn_rank_forward_noalloc(cp_attn_plan_t h, const void* q, const void* k, const void* v, void* out,
                                 float* lse, int rank, void* stream) {
  CPA_GUARD_BEGIN
  CPA_TRY(check_plan(h));
  Plan& p = *h->p;
  if (rank < 0 || rank >= p.cp) return fail(CP_ATTN_EINVAL, "rank outside [0, cp_size)");
  CPA_TRY(check_io(q, k, v, out, lse));
  if (!p.doc_starts.empty())
    return fail(CP_ATTN_EUNSUPPORTED, "document masks need the plan's workspace (cp_attn_rank_forward)");
  const int64_t need = ws_layout(p).total;
  if (need > kScratchBytes)
    return fail(CP_ATTN_ENOWORKSPACE, "the plan needs " + std::to_string(need) + " bytes of workspace; the " +
                                          "no-allocation forward holds " + std::to_string(kScratchBytes));
  DeviceState& d = *p.dev;
  int dev = 0;
  CPA_HIP(hipGetDevice(&dev));
  if (d.device >= 0 && d.device != dev) return fail(CP_ATTN_EINVAL, "plan was first used on another device");
  if (!d.cus) CPA_HIP(hipDeviceGetAttribute(&d.cus, hipDeviceAttributeMultiprocessorCount, dev));
  char* base = nullptr;
  CPA_TRY(scratch_base(dev, &base));
  d.device = dev;
  std::fill(d.timed.begin(), d.timed.end(), 0);  // this call records no step times or counts
  std::fill(d.counted.begin(), d.counted.end(), 0);
  RunCfg c;
  c.ws = base;
  c.serial = true;
  c.recv = 2;
  c.recv_blocks = p.opt_recv_blocks < 0 ? 256 : p.opt_recv_blocks;
  c.poison = p.opt_poison != 0;
  return run_rank(p, c, q, k, v, out, lse, rank, static_cast<hipStream_t>(stream));
  CPA_GUARD_END
}

int cp_attn_full_forward(cp_attn_plan_t h, const void* q, const void* k, const void* v, void* out, float* lse,
                         void* stream) {
  CPA_GUARD_BEGIN
  CPA_TRY(check_plan(h));
  Plan& p = *h->p;
  CPA_TRY(check_io(q, k, v, out, lse));
  CPA_TRY(ensure_device(p));
  reset_timing(p);
  if (p.opt_graph) return run_graph(p, q, k, v, out, lse, -1, static_cast<hipStream_t>(stream));
  const RunCfg c = plan_cfg(p, false);
  if (lockstep_served(p, c)) return run_lockstep(p, c, q, k, v, out, lse, static_cast<hipStream_t>(stream));
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (fused_ring_served(p, c)) {
    CPA_TRY(ensure_fused_ring(p));
    DeviceState& d = *p.dev;
    if (d.fr_ok && d.fr_lanes) {
      // two lanes: even ranks on the caller's stream, odd ranks on the
      // second lane, which starts behind the caller's earlier work and
      // which the caller's stream waits for at the end; a rank's launch then
      // runs beside its neighbour's, filling the compute units each leaves
      // idle at its end (results: the same bits as one rank at a time)
      CPA_TRY(ensure_fused_lane(p));
      CPA_HIP(hipEventRecord(d.fl_enter, st));
      CPA_HIP(hipStreamWaitEvent(d.fl_comp, d.fl_enter, 0));
      for (int r = 0; r < p.cp; ++r) {
        if (p.valid_rows(r) == 0) continue;
        CPA_TRY(run_rank_fused(p, c, q, k, v, out, lse, r, (r & 1) ? d.fl_comp : st, r & 1));
      }
      CPA_HIP(hipEventRecord(d.fl_join, d.fl_comp));
      CPA_HIP(hipStreamWaitEvent(st, d.fl_join, 0));
      return CP_ATTN_OK;
    }
  }
  for (int r = 0; r < p.cp; ++r) CPA_TRY(run_rank(p, c, q, k, v, out, lse, r, st));
  return CP_ATTN_OK;
  CPA_GUARD_END
}

int cp_attn_rank_backward(cp_attn_plan_t h, const void* q, const void* k, const void* v, const void* out,
                          const float* lse, const void* dout, float* dq, float* dk, float* dv, int rank,
                          void* stream) {
  CPA_GUARD_BEGIN
  CPA_TRY(check_plan(h));
  Plan& p = *h->p;
  if (rank < 0 || rank >= p.cp) return fail(CP_ATTN_EINVAL, "rank outside [0, cp_size)");
  CPA_TRY(check_io(q, k, v, out, lse));
  CPA_TRY(check_bwd_io(dout, dq, dk, dv));
  CPA_TRY(ensure_device(p));
  return run_rank_backward(p, q, k, v, out, lse, dout, dq, dk, dv, rank, static_cast<hipStream_t>(stream));
  CPA_GUARD_END
}

int cp_attn_full_backward(cp_attn_plan_t h, const void* q, const void* k, const void* v, const void* out,
                          const float* lse, const void* dout, float* dq, float* dk, float* dv, void* stream) {
  CPA_GUARD_BEGIN
  CPA_TRY(check_plan(h));
  Plan& p = *h->p;
  CPA_TRY(check_io(q, k, v, out, lse));
  CPA_TRY(check_bwd_io(dout, dq, dk, dv));
  CPA_TRY(ensure_device(p));
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t words = p.seq_len * p.heads * p.head_dim;
  CPA_HIP(launch_fill_words(dk, words, 0u, st));
  CPA_HIP(launch_fill_words(dv, words, 0u, st));
  for (int r = 0; r < p.cp; ++r) CPA_TRY(run_rank_backward(p, q, k, v, out, lse, dout, dq, dk, dv, r, st));
  return CP_ATTN_OK;
  CPA_GUARD_END
}

int cp_attn_local_rows(cp_attn_plan_t h, int64_t* rows) {
  CPA_TRY(check_plan(h));
  if (!rows) return fail(CP_ATTN_EINVAL, "rows is null");
  *rows = h->p->n_loc;
  return CP_ATTN_OK;
}

int cp_attn_rank_valid_rows(cp_attn_plan_t h, int rank, int64_t* rows) {
  CPA_TRY(check_plan(h));
  const Plan& p = *h->p;
  if (rank < 0 || rank >= p.cp) return fail(CP_ATTN_EINVAL, "rank outside [0, cp_size)");
  if (!rows) return fail(CP_ATTN_EINVAL, "rows is null");
  *rows = p.valid_rows(rank);
  return CP_ATTN_OK;
}

int cp_attn_rank_chunks(cp_attn_plan_t h, int rank, int32_t chunks[2], int32_t* count) {
  CPA_TRY(check_plan(h));
  const Plan& p = *h->p;
  if (!chunks || !count) return fail(CP_ATTN_EINVAL, "output is null");
  if (rank < 0 || rank >= p.cp) return fail(CP_ATTN_EINVAL, "rank outside [0, cp_size)");
  *count = p.layout == 1 ? 2 : 1;
  chunks[0] = int32_t(p.chunk_of(rank, 0));
  chunks[1] = p.layout == 1 ? int32_t(p.chunk_of(rank, 1)) : -1;
  return CP_ATTN_OK;
}

int cp_attn_step_source(cp_attn_plan_t h, int rank, int step, int32_t* source) {
  CPA_TRY(check_plan(h));
  const Plan& p = *h->p;
  if (!source) return fail(CP_ATTN_EINVAL, "source is null");
  if (rank < 0 || rank >= p.cp || step < 0 || step >= p.cp) return fail(CP_ATTN_EINVAL, "rank or step out of range");
  *source = p.step(rank, step).src;
  return CP_ATTN_OK;
}

int cp_attn_step_segments(cp_attn_plan_t h, int rank, int step, int64_t out[14], int32_t* count) {
  CPA_TRY(check_plan(h));
  const Plan& p = *h->p;
  if (!out || !count) return fail(CP_ATTN_EINVAL, "output is null");
  if (rank < 0 || rank >= p.cp || step < 0 || step >= p.cp) return fail(CP_ATTN_EINVAL, "rank or step out of range");
  const StepDesc& d = p.step(rank, step);
  *count = d.nseg;
  for (int i = 0; i < 2; ++i) {
    const Segment g = i < d.nseg ? d.seg[i] : Segment{};
    int64_t* o = out + 7 * i;
    o[0] = g.q_start;
    o[1] = g.q_len;
    o[2] = g.kv_full;
    o[3] = g.diag;
    o[4] = g.first;
    o[5] = g.last;
    o[6] = g.q_global;
  }
  return CP_ATTN_OK;
}

int cp_attn_valid_work(cp_attn_plan_t h, int rank, int step, int bm, int bn, int64_t* tiles, int64_t* pairs) {
  CPA_TRY(check_plan(h));
  const Plan& p = *h->p;
  if (rank < 0 || rank >= p.cp || step < 0 || step >= p.cp) return fail(CP_ATTN_EINVAL, "rank or step out of range");
  if (bm <= 0 || bn <= 0) return fail(CP_ATTN_EINVAL, "tile sizes must be positive");
  if (tiles) *tiles = step_tiles(p, rank, step, bm, bn);
  if (pairs) *pairs = step_pairs(p, rank, step);
  return CP_ATTN_OK;
}

static int layout_all(cp_attn_plan_t h, const void* src, void* dst, void* stream, int to_local) {
  CPA_TRY(check_plan(h));
  const Plan& p = *h->p;
  if (!src || !dst) return fail(CP_ATTN_EINVAL, "src or dst is null");
  if (!aligned16(src) || !aligned16(dst)) return fail(CP_ATTN_EINVAL, "src or dst not 16-byte aligned");
  LayoutArgs la{};
  la.src[0] = src;
  la.dst[0] = dst;
  la.ntensors = 1;
  la.rank_begin = 0;
  la.rank_count = p.cp;
  la.cp = p.cp;
  la.zigzag = p.layout == 1;
  la.to_local = to_local;
  la.chunk = p.chunk;
  la.n_loc = p.n_loc;
  la.row_vec = int64_t(p.heads) * p.head_dim * p.elem_bytes() / 16;
  la.seq_len = p.seq_len;
  la.dst_rank0 = 0;
  CPA_HIP(launch_layout(la, 0, static_cast<hipStream_t>(stream)));
  return CP_ATTN_OK;
}

int cp_attn_layout_gather(cp_attn_plan_t h, const void* src, void* dst, void* stream) {
  return layout_all(h, src, dst, stream, 1);
}

int cp_attn_layout_scatter(cp_attn_plan_t h, const void* src, void* dst, void* stream) {
  return layout_all(h, src, dst, stream, 0);
}

int cp_attn_lse_merge(float* o_acc, float* lse_acc, const float* o_s, const float* lse_s, int64_t rows, int heads,
                      int head_dim, void* stream) {
  if (!o_acc || !lse_acc || !o_s || !lse_s) return fail(CP_ATTN_EINVAL, "null pointer");
  if (!aligned16(o_acc) || !aligned16(o_s)) return fail(CP_ATTN_EINVAL, "O pointers not 16-byte aligned");
  if (rows < 0 || heads <= 0 || head_dim <= 0 || head_dim % 4 || 64 % (head_dim / 4) || rows > INT32_MAX)
    return fail(CP_ATTN_EINVAL, "bad sizes (head_dim/4 must divide 64)");
  if (rows == 0) return CP_ATTN_OK;
  MergeArgs m{};
  m.o_s = o_s;
  m.lse_s = lse_s;
  m.o_acc = o_acc;
  m.lse_acc = lse_acc;
  m.n_rows_total = rows;
  m.heads = heads;
  m.head_dim = head_dim;
  m.nseg = 1;
  m.seg_start[0] = 0;
  m.seg_len[0] = int32_t(rows);
  CPA_HIP(launch_merge(m, static_cast<hipStream_t>(stream)));
  return CP_ATTN_OK;
}

int cp_attn_last_tile_counts(cp_attn_plan_t h, int64_t* counts, int n, int32_t* tile_rows, int32_t* tile_keys) {
  CPA_TRY(check_plan(h));
  const Plan& p = *h->p;
  if (!counts) return fail(CP_ATTN_EINVAL, "counts is null");
  const size_t nn = size_t(p.cp) * p.cp;
  if (n < 0 || size_t(n) < nn) return fail(CP_ATTN_EINVAL, "n < cp_size * cp_size");
  const bool bf16 = p.dtype == CP_ATTN_BF16;
  if (tile_rows) *tile_rows = bf16 ? 32 : attn_f32_block_m();
  if (tile_keys) *tile_keys = bf16 ? 64 : attn_f32_block_n();
  DeviceState& d = *p.dev;
  for (size_t i = 0; i < nn; ++i) counts[i] = -1;
  if (!d.tile_cnt) return CP_ATTN_OK;
  std::vector<unsigned long long> c(nn);
  CPA_HIP(hipDeviceSynchronize());
  CPA_HIP(hipMemcpy(c.data(), d.tile_cnt, nn * sizeof(unsigned long long), hipMemcpyDeviceToHost));
  for (size_t i = 0; i < nn; ++i)
    if (i < d.counted.size() && d.counted[i]) counts[i] = int64_t(c[i]);
  return CP_ATTN_OK;
}

int cp_attn_last_step_times(cp_attn_plan_t h, float* ms, int n) {
  CPA_TRY(check_plan(h));
  const Plan& p = *h->p;
  if (!ms) return fail(CP_ATTN_EINVAL, "ms is null");
  const size_t nn = size_t(p.cp) * p.cp;
  if (n < 0 || size_t(n) < nn) return fail(CP_ATTN_EINVAL, "n < cp_size * cp_size");
  DeviceState& d = *p.dev;
  for (size_t i = 0; i < nn; ++i) {
    ms[i] = -1.f;
    if (i < d.timed.size() && d.timed[i] && i < d.t1.size()) {
      CPA_HIP(hipEventSynchronize(d.t1[i]));
      float t = 0.f;
      CPA_HIP(hipEventElapsedTime(&t, d.t0[i], d.t1[i]));
      ms[i] = t;
    }
  }
  return CP_ATTN_OK;
}

const char* cp_attn_status_string(int status) {
  switch (status) {
    case CP_ATTN_OK:
      return "ok";
    case CP_ATTN_EINVAL:
      return "invalid argument";
    case CP_ATTN_EUNSUPPORTED:
      return "unsupported configuration";
    case CP_ATTN_ENOWORKSPACE:
      return "workspace missing, too small or not allocatable";
    case CP_ATTN_EHIP:
      return "HIP runtime error";
    default:
      return "unknown status";
  }
}

const char* cp_attn_last_error(void) { return g_err.c_str(); }

}  // extern "C"
