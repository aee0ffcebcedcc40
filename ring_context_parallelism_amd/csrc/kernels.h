// Kernel argument structs and launcher declarations shared by the HIP
// translation units of libcpattn.so (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace cpattn {

// Epilogue of a step for one row segment.
enum EpiMode : int32_t {
  kEpiInit = 0,     // running state := this step's partial
  kEpiMerge = 1,    // running state := LSE-merge(running state, partial)
  kEpiPartial = 2,  // write the partial to the partial buffer (separate merge)
};
constexpr int32_t kEpiFinal = 4;  // with Init/Merge: write the result to out/lse instead of the state

struct SegArgs {
  int64_t q_global;  // global token of local row q_start
  int32_t q_start;   // first local row
  int32_t q_len;     // rows
  int32_t kv_full;   // keys every row sees
  int32_t diag;      // 1: row t also sees keys kv_full .. kv_full + t
  int32_t epi;       // EpiMode | kEpiFinal
  int32_t tiles;     // workgroups of the segment: ceil(q_len / BM) * ksplit
  int32_t ksplit;    // 1, or 2: each row tile's keys in two halves, one workgroup each (full segments
                     // starting at a multiple of 256 local rows only)
  int32_t run0;      // fused ring: index in StepArgs::runs of the segment's first key run
};

// Fused ring (every ring step of a rank in one launch): the keys a segment's
// rows see are a sequence of runs, in the order the workgroup takes them.
// Run i covers the segment's keys [end of run i-1, end) and key kk of it is
// source row kk + delta of buffer buf (0: the rank's own natural-order K/V,
// 1: the receive slots); its rows are there once flag `step` of the call has
// reached the call's epoch (step < 0: nothing to wait for).
struct RingRun {
  int32_t end;
  int32_t delta;
  int32_t buf;
  int32_t step;
};

// Ring receive: up to four contiguous byte ranges (16-byte multiples).
struct RecvArgs {
  const void* src[4];
  void* dst[4];
  int64_t vec[4];  // 16-byte vectors per range
  int32_t n;
};

struct StepArgs {
  const void* q;     // [S][H][D] natural order, plan dtype
  // K/V source: rows of [H][D] elements.  Local key kk (0 <= kk < n_loc) is
  // row kv_lo + kk if kk < kv_split, else row kv_hi + (kk - kv_split).  A
  // receive slot is (0, split, split); the rank's own chunks are read in
  // place from the natural-order tensors.
  const void* k;
  const void* v;
  int64_t kv_bytes;  // bytes addressable from k and from v
  int32_t kv_lo;
  int32_t kv_hi;
  int32_t kv_split;
  float* acc_o;      // [n_loc][H][D] running O (normalised)
  float* acc_lse;    // [H][n_loc] running LSE (natural log)
  float* part_o;     // [n_loc][H][D] partial O (separate merge mode)
  float* part_lse;   // [H][n_loc]
  void* out;         // [S][H][D] plan dtype
  float* lse;        // [H][S]
  int64_t seq_len;
  int32_t n_loc;
  int32_t kv_valid;  // real keys of the source: local keys [0, kv_valid); loads never go past them
  int32_t heads;
  float scale_log2;  // softmax scale * log2(e)
  float scale;       // softmax scale 1/sqrt(D)
  int32_t out_f32;   // 1: out is fp32, 0: bf16
  int32_t nseg;
  int32_t total_tiles;  // sum of seg[i].tiles, i < nseg
  // seg[2], seg[3]: fused ring only, part 1 of a key-split seg[0], seg[1]
  // (the same rows; its own run list and kv_full, the diagonal if any);
  // seg[0], seg[1] then describe part 0 (the first half of every full run)
  SegArgs seg[4];
  RecvArgs recv;        // next step's receive done by this kernel (recv.n == 0: none)
  // key split (segments with ksplit 2): part p of the 256-row tile r (of the
  // local rows) and head h leaves its normalised output in the 128 KiB slot
  // r * heads + h of split_o[p] (n_loc * H * D floats, n_loc a multiple of
  // 256) and its LSE in split_lse[p]; split_cnt holds one counter per slot,
  // zero between launches
  float* split_o[2];
  float* split_lse[2];
  int32_t* split_cnt;
  // work counter (null: off): the kernel adds the key tiles it computed, per
  // wave of 32 rows x 64 keys (bf16 kernels) or per workgroup tile (fp32)
  unsigned long long* tile_cnt;
  // document masks (null: none): doc[2 p], doc[2 p + 1] = [start, end) of the
  // document holding global position p.  Local key kk of the source sits at
  // global position kpos_lo + kk below kpos_split, kpos_hi + kk - kpos_split
  // from there on; a row sees only the keys of its own document.
  const int32_t* doc;
  int32_t kpos_lo;
  int32_t kpos_hi;
  int32_t kpos_split;
  // fused ring (null runs: not fused): the receive slots of steps 1 .. P-1,
  // K and V each one buffer of rows (kv2_bytes addressable from each), the
  // segments' key runs, and the per-step receive flags; the call's epoch is
  // ring_flags[0] plus ring_epoch_add (under graph capture word 0 is
  // advanced by a kernel before the launch and the addend is 0; otherwise
  // word 0 stays 0 and the host passes the epoch as the addend), flag s is
  // done once it reaches that epoch; a workgroup polls
  // flag s (at most ring_polls times) before it loads any row of a run of
  // step s, and a wait that runs out stores 1 to *ring_err (host-visible)
  const void* k2;
  const void* v2;
  int64_t kv2_bytes;
  const RingRun* runs;
  const uint32_t* ring_flags;
  uint32_t* ring_err;
  uint32_t ring_epoch_add;
  int32_t ring_polls;
};

// Backward of one ring step (attn_bwd.hip, attn_bwd_bf16.hip).  Q, dO, O are
// read at the natural rows of the segments, K and V of the source in place
// through the two-run map (local key kk -> row kv_lo + kk below kv_split, else
// kv_hi + kk - kv_split); gradients are fp32 [S][H][D] at natural rows.
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* out;   // forward output (delta kernel)
  const void* dout;
  const float* lse;  // [H][S] forward LSE, natural log
  float* delta;      // [H][n_loc] D_i = <dO_i, O_i> of local row i
  float* dq;         // written at a row run's first step (SegArgs::epi != 0), added to later
  float* dk;         // added to
  float* dv;         // added to
  int64_t seq_len;
  int32_t n_loc;
  int32_t heads;
  int32_t kv_valid;
  int32_t kv_lo;
  int32_t kv_hi;
  int32_t kv_split;
  float scale;
  float scale_log2;
  int32_t nseg;
  int32_t total_tiles;  // row-major workgroups per head (sum of seg[i].tiles)
  int32_t key_tiles;    // key-major workgroups per head
  SegArgs seg[2];       // epi: 1 = first active step of the row run
  // delta kernel: the rank's real local rows, local row -> natural row map
  int64_t delta_rows;
  int64_t delta_lo;
  int64_t delta_hi;
  int64_t delta_split;
  // document masks, as in StepArgs (null: none)
  const int32_t* doc;
  int32_t kpos_lo;
  int32_t kpos_hi;
  int32_t kpos_split;
};
int bwd_generic_tile();  // rows and keys per workgroup of the generic kernels
hipError_t launch_bwd_delta(const BwdArgs& a, int dtype_bf16, int head_dim, hipStream_t stream);
hipError_t launch_bwd_generic(const BwdArgs& a, int dtype_bf16, int head_dim, hipStream_t stream);
bool bwd_mfma(int dtype_bf16, int head_dim);  // the matrix-core kernels serve this configuration
int bwd_mfma_rows();                          // rows per row-major workgroup
int bwd_mfma_keys();                          // keys per key-major workgroup
hipError_t launch_bwd_bf16_d128(const BwdArgs& a, bool eight_wave_keys, hipStream_t stream);

// attention step kernels: return hipError_t of the launch
// (only the head_dim 128 bf16 kernel performs StepArgs::recv)
bool attn_does_recv(int dtype_bf16, int head_dim);
bool attn_splits_keys(int dtype_bf16, int head_dim);  // kernel honours SegArgs::ksplit
hipError_t launch_attn_bf16(const StepArgs& a, int head_dim, hipStream_t stream);
// fused ring: one launch of the bf16 head_dim 128 kernel over every ring step
// of a rank (StepArgs::runs set)
hipError_t launch_attn_bf16_ring(const StepArgs& a, hipStream_t stream);
// store *epoch to *flag (release, agent scope) from one thread, once every
// kernel before it on the stream has completed
hipError_t launch_ring_signal(uint32_t* flag, const uint32_t* epoch, hipStream_t stream);
// the same with the epoch by value
hipError_t launch_ring_signal_value(uint32_t* flag, uint32_t epoch, hipStream_t stream);
// advance the epoch word by one (never to zero), one thread
hipError_t launch_ring_epoch(uint32_t* epoch, hipStream_t stream);
// Every rank's step of one ring step in one launch (bf16, head_dim 128, no
// in-kernel receive): tbl[r] (device memory) are rank r's arguments, its
// workgroups wgb[r] .. wgb[r + 1] - 1 (wgb[nranks] = total_wgs; each range
// starts at a multiple of 8 and holds at least tbl[r].total_tiles * heads).
hipError_t launch_attn_bf16_ranks(const StepArgs* tbl, const int32_t* wgb, int nranks, int total_wgs, bool doc,
                                  hipStream_t stream);
hipError_t launch_attn_f32(const StepArgs& a, int head_dim, hipStream_t stream);
int attn_bf16_block_m(int head_dim);
int attn_f32_block_m();
int attn_f32_block_n();

// Row copies between natural order and rank-local order.
//   gather (to_local=1): dst row (rank_begin+i)*n_loc + li  <-  src global_row(rank, li)
//   scatter (to_local=0): the inverse.  ntensors (1 or 2) pairs src/dst.
struct LayoutArgs {
  const void* src[2];
  void* dst[2];
  int32_t ntensors;
  int32_t rank_begin;
  int32_t rank_count;
  int32_t cp;
  int32_t zigzag;
  int32_t to_local;
  int64_t chunk;       // rows per chunk
  int64_t n_loc;       // rows per rank
  int64_t row_vec;     // 16-byte vectors per row
  int64_t seq_len;     // real tokens: pad rows (token >= seq_len) are zero-filled by gather, skipped by scatter
  int64_t dst_rank0;   // rank whose local buffer starts at dst (gather) / src (scatter) row 0
};
// max_blocks > 0 bounds the grid (per tensor); 0 sizes it to the data.
hipError_t launch_layout(const LayoutArgs& a, int max_blocks, hipStream_t stream);

hipError_t launch_recv(const RecvArgs& a, int blocks, hipStream_t stream);

// Ulysses all-to-all of every rank at once (one GPU): sequence ownership
// [cp][n_loc][H][D] (each rank's rows in its local order) <-> head ownership
// [cp][S][H/cp][D] (rank r: every token of heads r H/cp .. (r+1) H/cp - 1).
struct UlyssesArgs {
  const void* src;
  void* dst;
  int32_t to_heads;  // 1: sequence -> head ownership, 0: back (pad rows of the sequence layout untouched)
  int32_t cp;
  int32_t zigzag;
  int64_t seq_len;   // real tokens
  int64_t chunk;     // rows per chunk
  int64_t n_loc;     // rows per rank in the sequence layout
  int64_t heads;
  int64_t head_vec;  // 16-byte vectors per head row (head_dim * element size / 16)
};
hipError_t launch_ulysses(const UlyssesArgs& a, hipStream_t stream);

// Fill with NaN (all-ones bytes) -- a kernel, not a memset, so it is safe in captured graphs.
hipError_t launch_poison(void* ptr, int64_t bytes, hipStream_t stream);
hipError_t launch_fill_words(void* ptr, int64_t words, uint32_t value, hipStream_t stream);

// Separate LSE merge (part -> acc) for up to two row segments, optionally
// writing the final output.  rows_* are local rows.
struct MergeArgs {
  const float* o_s;
  const float* lse_s;
  float* o_acc;
  float* lse_acc;
  int64_t n_rows_total;  // row stride of the lse arrays
  int32_t heads;
  int32_t head_dim;
  int32_t nseg;
  int32_t seg_start[2];
  int32_t seg_len[2];
};
hipError_t launch_merge(const MergeArgs& a, hipStream_t stream);

// Finalize: running state -> out (plan dtype, RNE) and lse at global rows.
struct FinalizeArgs {
  const float* acc_o;
  const float* acc_lse;
  void* out;
  float* lse;
  int64_t seq_len;
  int32_t n_loc;
  int32_t heads;
  int32_t head_dim;
  int32_t out_f32;
  int32_t nseg;
  int32_t seg_start[2];
  int32_t seg_len[2];
  int64_t seg_global[2];
};
hipError_t launch_finalize(const FinalizeArgs& a, hipStream_t stream);

}  // namespace cpattn
