// Host-side plan for zigzag / contiguous ring context-parallel attention.
//
// Chunk placement follows "Sequence Parallelism IV: Megatron Context Parallel
// and Load-Balanced Rings", section 3 (Naive Ring Attention Is Imbalanced
// Under Causal Masks): 2*cp chunks, rank r owns the early chunk r and the late
// chunk 2*cp-1-r, kept early first in the rank's local buffer; the naive
// placement gives rank r the contiguous slice r.  The ring (sections 4 and 5)
// moves K/V to a neighbour each step; rank r receives from r-1, so at step s
// it holds the K/V of source j = (r - s) mod cp.
//
// Causal step descriptors (section 4: a step's mask is decided by the global
// positions of the rank's own queries and of the visiting keys, and key
// blocks wholly in a query block's future are not computed).  For a query chunk a and key chunk b of equal length, the pair is
// fully visible if b < a, causal on the diagonal if b == a, and skipped if
// b > a.  With a in {r, 2cp-1-r} and b in {j, 2cp-1-j}:
//   j == r : (r, r) diagonal; (2cp-1-r, r) full; (2cp-1-r, 2cp-1-r) diagonal;
//            (r, 2cp-1-r) skipped -- causal over the local buffer.
//   j <  r : both query chunks see key chunk j fully and skip 2cp-1-j.
//   j >  r : query chunk r sees nothing; chunk 2cp-1-r sees both key chunks.
// In every case a local row's valid keys form a prefix of the source's local
// buffer, which is what a Segment records.
//
// Document masks ("Context Parallelism for Long-Context Training", section
// "Prove attention equivalence": causal and document masks) leave the
// descriptors as they are: a document is a run of positions and a source's
// local keys are in increasing position order, so the keys of a row's
// document are one run of the source's local buffer, [keys_before(start),
// keys_before(end)); a row sees that run clipped to its prefix.
//
// Awkward lengths ("Context Parallelism for Long-Context Training", section
// "Test sequence divisibility and padding": pad ownership, masked pad keys and
// queries, local offsets).  A length that does not divide into the chunks is
// padded at the end to the next multiple; pad token c*chunk + i belongs to the
// owner of chunk c like any other.  Chunk c holds vl(c) = clamp(S - c*chunk, 0,
// chunk) real tokens, first.  A chunk with a real token has only real chunks
// before it, so a rank's real rows are a prefix of its local buffer (its early
// chunk is full whenever its late chunk holds anything), and so are a
// source's real keys.  Segments keep only real rows; causal rows only ever
// see keys before them, which are real; bidirectional rows see the source's
// real prefix.  Pad rows appear in no segment and pad keys in no prefix.
#include "plan.h"

#include <algorithm>

namespace cpattn {

namespace {
constexpr int kOk = 0, kInval = -1, kUnsupported = -2;
}

int64_t Plan::chunk_of(int r, int which) const {
  if (layout == 0) return r;
  return which == 0 ? r : 2 * int64_t(cp) - 1 - r;
}

int64_t Plan::global_row(int r, int64_t i) const {
  if (layout == 0) return int64_t(r) * chunk + i;
  int which = i < chunk ? 0 : 1;
  return chunk_of(r, which) * chunk + (i - which * chunk);
}

int64_t Plan::valid_in_chunk(int64_t c) const { return std::min(chunk, std::max<int64_t>(0, seq_len - c * chunk)); }

int64_t Plan::valid_rows(int r) const {
  if (layout == 0) return valid_in_chunk(r);
  return valid_in_chunk(chunk_of(r, 0)) + valid_in_chunk(chunk_of(r, 1));
}

void Plan::doc_range(int64_t pos, int64_t* start, int64_t* end) const {
  if (doc_starts.empty()) {
    *start = 0;
    *end = seq_len;
    return;
  }
  const auto it = std::upper_bound(doc_starts.begin(), doc_starts.end(), pos);  // first start after pos
  *start = *(it - 1);
  *end = it == doc_starts.end() ? seq_len : *it;
}

int64_t Plan::keys_before(int j, int64_t pos) const {
  auto run = [&](int64_t first, int64_t len) { return std::min(len, std::max<int64_t>(0, pos - first)); };
  if (layout == 0) return run(int64_t(j) * chunk, chunk);
  return run(chunk_of(j, 0) * chunk, chunk) + run(chunk_of(j, 1) * chunk, chunk);
}

namespace {
void row_keys(const Plan& p, const StepDesc& d, const Segment& g, int64_t t, int64_t* lo, int64_t* hi);
}
static void build_steps(Plan& p);
static void mark_first_last(Plan& p);

int set_documents(Plan& p, const int64_t* starts, int64_t count, std::string* err) {
  if (count < 0 || (count > 0 && !starts)) {
    *err = "documents: count < 0, or starts is null";
    return kInval;
  }
  for (int64_t d = 0; d < count; ++d) {
    if ((d == 0 && starts[0] != 0) || (d > 0 && starts[d] <= starts[d - 1]) || starts[d] >= p.seq_len) {
      *err = "documents: starts must increase strictly from 0 and stay below seq_len";
      return kInval;
    }
  }
  p.doc_starts.assign(starts, starts + count);
  ++p.doc_version;
  build_steps(p);
  if (!p.doc_starts.empty()) {
    // a segment none of whose rows sees a key of the step's source under the
    // documents is dropped, and the first / last steps of the row runs follow
    for (auto& d : p.steps) {
      int kept = 0;
      for (int i = 0; i < d.nseg; ++i) {
        bool any = false;
        for (int64_t t = 0; t < d.seg[i].q_len && !any; ++t) {
          int64_t lo = 0, hi = 0;
          row_keys(p, d, d.seg[i], t, &lo, &hi);
          any = hi > lo;
        }
        if (any) d.seg[kept++] = d.seg[i];
      }
      d.nseg = kept;
    }
    mark_first_last(p);
  }
  return kOk;
}

static void build_steps(Plan& p) {
  const int P = p.cp;
  const int64_t C = p.chunk;
  p.steps.assign(size_t(P) * P, StepDesc{});
  for (int r = 0; r < P; ++r) {
    // real rows of the rank's early / late chunk
    const int64_t q0 = p.valid_in_chunk(p.chunk_of(r, 0));
    const int64_t q1 = p.layout == 1 ? p.valid_in_chunk(p.chunk_of(r, 1)) : 0;
    for (int s = 0; s < P; ++s) {
      StepDesc& d = p.steps[size_t(r) * P + s];
      const int j = ((r - s) % P + P) % P;
      d.src = j;
      // a segment with no real row, or whose rows see no key, is dropped
      auto add = [&](int64_t q_start, int64_t q_len, int64_t kv_full, int diag) {
        if (q_len <= 0 || (kv_full <= 0 && !diag)) return;
        Segment& g = d.seg[d.nseg++];
        g.q_start = q_start;
        g.q_len = q_len;
        g.kv_full = kv_full;
        g.diag = diag;
        g.q_global = p.global_row(r, q_start);
      };
      if (p.layout == 1) {  // zigzag: local rows [0,C) chunk r, [C,2C) chunk 2P-1-r
        if (!p.causal) {
          const int64_t kv = p.valid_rows(j);  // the source's real keys
          add(0, q0, kv, 0);
          add(C, q1, kv, 0);
        } else if (j == r) {
          add(C, q1, C, 1);  // late chunk first: the longer rows (longest-first order)
          add(0, q0, 0, 1);
        } else if (j < r) {
          add(0, q0, C, 0);
          add(C, q1, C, 0);
        } else {
          add(C, q1, 2 * C, 0);
        }
      } else {  // contiguous: local rows [0,L) chunk r
        if (!p.causal) {
          add(0, q0, p.valid_rows(j), 0);
        } else if (j == r) {
          add(0, q0, 0, 1);
        } else if (j < r) {
          add(0, q0, C, 0);
        }
      }
    }
  }
  mark_first_last(p);
}

// first / last active step of each row run (identified by q_start)
static void mark_first_last(Plan& p) {
  const int P = p.cp;
  for (int r = 0; r < P; ++r) {
    for (int s = 0; s < P; ++s) {
      StepDesc& d = p.steps[size_t(r) * P + s];
      for (int i = 0; i < d.nseg; ++i) {
        Segment& g = d.seg[i];
        int first = s, last = s;
        for (int t = 0; t < P; ++t) {
          const StepDesc& e = p.steps[size_t(r) * P + t];
          for (int k = 0; k < e.nseg; ++k) {
            if (e.seg[k].q_start == g.q_start) {
              first = std::min(first, t);
              last = std::max(last, t);
            }
          }
        }
        g.first = (first == s);
        g.last = (last == s);
      }
    }
  }
}

int make_plan(int64_t seq_len, int cp, int heads, int head_dim, int causal, int layout, Plan** out,
              std::string* err) {
  if (!out) {
    *err = "out is null";
    return kInval;
  }
  *out = nullptr;
  if (seq_len <= 0 || cp <= 0 || heads <= 0 || head_dim <= 0) {
    *err = "seq_len, cp_size, heads and head_dim must be positive";
    return kInval;
  }
  if (causal != 0 && causal != 1) {
    *err = "causal must be 0 or 1";
    return kInval;
  }
  if (layout != 0 && layout != 1) {
    *err = "layout must be CP_ATTN_CONTIGUOUS or CP_ATTN_ZIGZAG";
    return kInval;
  }
  if (cp > 256) {
    *err = "cp_size above 256 is not supported";
    return kUnsupported;
  }
  const int64_t parts = layout == 1 ? 2 * int64_t(cp) : int64_t(cp);
  const int64_t padded = (seq_len + parts - 1) / parts * parts;
  if (head_dim != 64 && head_dim != 128) {
    *err = "head_dim must be 64 or 128";
    return kUnsupported;
  }
  // The kernels address one rank's rows (a receive slot, a segment, the
  // fp32 running state) with 32-bit byte offsets from a base, and token rows
  // with 32-bit integers; natural-order tensors are otherwise addressed with
  // 64-bit offsets (beyond 4 GiB of K/V, step 0 reads the rank's own chunks
  // from a receive slot rather than in place).
  if (padded / cp * int64_t(heads) * head_dim * 4 >= (int64_t(1) << 32)) {
    *err = "(padded seq_len / cp_size) * heads * head_dim * 4 must stay below 2^32 bytes";
    return kUnsupported;
  }
  if (padded >= (int64_t(1) << 31)) {
    *err = "padded seq_len must stay below 2^31";
    return kUnsupported;
  }
  Plan* p = new Plan;
  p->seq_len = seq_len;
  p->cp = cp;
  p->heads = heads;
  p->head_dim = head_dim;
  p->causal = causal;
  p->layout = layout;
  p->padded_len = padded;
  p->chunk = padded / parts;
  p->n_loc = padded / cp;
  build_steps(*p);
  *out = p;
  return kOk;
}

namespace {
// Local key run [lo, hi) that segment row t sees in step (r, s) under the
// document mask: its prefix clipped to its document's run of the source.
void row_keys(const Plan& p, const StepDesc& d, const Segment& g, int64_t t, int64_t* lo, int64_t* hi) {
  int64_t ds = 0, de = 0;
  p.doc_range(g.q_global + t, &ds, &de);
  *lo = p.keys_before(d.src, ds);
  *hi = std::min(g.kv_full + (g.diag ? t + 1 : 0), p.keys_before(d.src, de));
}
}  // namespace

int64_t step_pairs(const Plan& p, int r, int s) {
  const StepDesc& d = p.step(r, s);
  int64_t n = 0;
  if (!p.doc_starts.empty()) {
    for (int i = 0; i < d.nseg; ++i) {
      for (int64_t t = 0; t < d.seg[i].q_len; ++t) {
        int64_t lo = 0, hi = 0;
        row_keys(p, d, d.seg[i], t, &lo, &hi);
        n += std::max<int64_t>(0, hi - lo);
      }
    }
    return n;
  }
  for (int i = 0; i < d.nseg; ++i) {
    const Segment& g = d.seg[i];
    n += g.q_len * g.kv_full;
    if (g.diag) n += g.q_len * (g.q_len + 1) / 2;
  }
  return n;
}

int64_t step_tiles(const Plan& p, int r, int s, int bm, int bn) {
  const StepDesc& d = p.step(r, s);
  int64_t tiles = 0;
  if (!p.doc_starts.empty()) {
    // per row tile, the key tiles that some row's run reaches (a difference
    // array over key tiles)
    const int64_t nk = (p.n_loc + bn - 1) / bn;
    std::vector<int64_t> cover(size_t(nk) + 1);
    for (int64_t i0 = 0; i0 < p.n_loc; i0 += bm) {
      std::fill(cover.begin(), cover.end(), 0);
      const int64_t i1 = std::min<int64_t>(p.n_loc, i0 + bm);
      for (int k = 0; k < d.nseg; ++k) {
        const Segment& g = d.seg[k];
        for (int64_t i = std::max(i0, g.q_start); i < std::min(i1, g.q_start + g.q_len); ++i) {
          int64_t lo = 0, hi = 0;
          row_keys(p, d, g, i - g.q_start, &lo, &hi);
          if (hi <= lo) continue;
          ++cover[size_t(lo / bn)];
          --cover[size_t((hi + bn - 1) / bn)];
        }
      }
      int64_t run = 0;
      for (int64_t kt = 0; kt < nk; ++kt) {
        run += cover[size_t(kt)];
        tiles += run > 0;
      }
    }
    return tiles;
  }
  for (int64_t i0 = 0; i0 < p.n_loc; i0 += bm) {
    const int64_t i1 = std::min<int64_t>(p.n_loc, i0 + bm);
    int64_t maxpre = 0;  // longest valid key prefix among the tile's rows
    for (int k = 0; k < d.nseg; ++k) {
      const Segment& g = d.seg[k];
      const int64_t a = std::max(i0, g.q_start), b = std::min(i1, g.q_start + g.q_len);
      if (a >= b) continue;
      const int64_t pre = g.kv_full + (g.diag ? (b - 1 - g.q_start) + 1 : 0);
      maxpre = std::max(maxpre, pre);
    }
    tiles += (maxpre + bn - 1) / bn;
  }
  return tiles;
}

}  // namespace cpattn
