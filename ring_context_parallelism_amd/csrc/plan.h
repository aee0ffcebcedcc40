// Host-side plan: chunk map, ring sources and per-(rank, step) descriptors.
// Pure C++ (no HIP), so it builds with any host compiler.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

namespace cpattn {

// One run of local query rows that all see a prefix of the source's local
// K/V buffer: local row q_start + t sees keys [0, kv_full + (diag ? t + 1 : 0)).
struct Segment {
  int64_t q_start = 0;
  int64_t q_len = 0;
  int64_t kv_full = 0;
  int32_t diag = 0;
  int32_t first = 0;  // first ring step in which these rows are active
  int32_t last = 0;   // last ring step in which these rows are active
  int64_t q_global = 0;  // global token position of local row q_start
};

struct StepDesc {
  int32_t src = 0;
  int32_t nseg = 0;
  Segment seg[2];
};

struct DeviceState;  // streams, events, workspace (defined with the HIP code)

struct Plan {
  int64_t seq_len = 0;
  int32_t cp = 1;
  int32_t heads = 0;
  int32_t head_dim = 0;
  int32_t causal = 1;
  int32_t layout = 1;
  int32_t dtype = 0;
  int64_t padded_len = 0;  // seq_len rounded up to a multiple of the chunk count
  int64_t chunk = 0;   // padded_len/(2cp) zigzag, padded_len/cp contiguous
  int64_t n_loc = 0;   // rows of a rank's local buffer (pad rows included)
  std::vector<StepDesc> steps;  // [rank * cp + step]
  // document masks: document d holds positions [doc_starts[d], doc_starts[d+1])
  // (the last runs to seq_len); empty = one document (no document mask)
  std::vector<int64_t> doc_starts;
  int64_t doc_version = 0;  // bumped by every change of doc_starts

  // options
  int32_t opt_merge = 0;
  int32_t opt_serialize = 0;
  int32_t opt_recv = 0;
  int32_t opt_poison = 0;
  int32_t opt_step_timing = 0;
  int32_t opt_graph = 0;
  int32_t opt_ksplit = 1;
  int32_t opt_counters = 0;
  int32_t opt_bwd_keys = 0;
  int32_t opt_lockstep = 0;
  int32_t opt_fused_ring = 1;
  int32_t opt_bwd_fused = 1;
  int32_t opt_recv_blocks = -1;  // -1: automatic (256 beside a step launch, 1024 beside the fused ring)

  DeviceState* dev = nullptr;

  const StepDesc& step(int r, int s) const { return steps[size_t(r) * cp + s]; }
  int64_t elem_bytes() const { return dtype == 1 ? 4 : 2; }
  // global token position of local row i of rank r
  int64_t global_row(int r, int64_t i) const;
  int64_t chunk_of(int r, int which) const;  // which in {0, 1}
  // real (non-pad) tokens of chunk c: the first valid_in_chunk(c) rows
  int64_t valid_in_chunk(int64_t c) const;
  // real rows of rank r's local buffer; they are its first valid_rows(r) rows
  int64_t valid_rows(int r) const;
  // [start, end) of the document holding global position pos (the whole
  // sequence when no documents are set)
  void doc_range(int64_t pos, int64_t* start, int64_t* end) const;
  // local keys of source j whose global position is below pos
  int64_t keys_before(int j, int64_t pos) const;
};

// Returns a status code; on success *out is a new plan.
int make_plan(int64_t seq_len, int cp, int heads, int head_dim, int causal, int layout, Plan** out,
              std::string* err);

// Checks and stores a document list (strictly increasing, first 0, all below
// seq_len; count 0 clears it).
int set_documents(Plan& p, const int64_t* starts, int64_t count, std::string* err);

int64_t step_pairs(const Plan& p, int r, int s);
int64_t step_tiles(const Plan& p, int r, int s, int bm, int bn);

}  // namespace cpattn
