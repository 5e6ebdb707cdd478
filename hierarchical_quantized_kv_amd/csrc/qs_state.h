// qs_state.h -- host-side bookkeeping of the cache: configuration checks, arena layout, the
// per-(layer, sequence) tail/quantized counters, validation of every verb before it mutates
// anything, and the work plan of an attention call.  Pure C++17: no HIP, so it is unit-tested
// on the CPU.
//
// The bookkeeping follows the double full-precision buffer of the QuantSpec Guide (section
// "3. Double Full-Precision Cache Buffer (CF1 and CF2)") and of the Pith review of
// arXiv:2502.10424 ("What carries the argument", "Core claim"): new tokens enter a 2G-slot fp16
// ring unquantized, rejected tokens leave it by rollback, and the oldest G-token half is
// quantized by a flush.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <string>
#include <vector>

#include "qs_args.h"

namespace qs {

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Checks a configuration; on failure writes the reason to *why.
inline bool config_ok(const qs_config& c, std::string* why) {
  auto fail = [&](const char* m) { if (why) *why = m; return false; };
  if (c.n_layers < 1) return fail("n_layers must be >= 1");
  if (c.batch < 1 || c.batch > QS_MAX_BATCH) return fail("batch must be in 1..QS_MAX_BATCH");
  if (c.n_heads < 1) return fail("n_heads must be >= 1");
  if (c.head_dim != 64 && c.head_dim != 128) return fail("head_dim must be 64 or 128");
  if (c.group != kGroup) return fail("group must be 128");
  if (c.max_ctx < c.group || c.max_ctx % c.group) return fail("max_ctx must be a positive multiple of group");
  if ((long long)c.max_ctx / c.group > (long long)kMaxQuantSplits * 1024) return fail("max_ctx too large");
  if (c.gamma_max < 0 || c.gamma_max + 1 > QS_MAX_QUERIES) return fail("gamma_max + 1 must be in 1..16");
  if (c.draft_offset != 0 && c.draft_offset != 8) return fail("draft_offset must be 0 or 8");
  if (c.meta_fp16 != 0 && c.meta_fp16 != 1) return fail("meta_fp16 must be 0 or 1");
  if (c.split_upper != 0 && c.split_upper != 1) return fail("split_upper must be 0 or 1");
  if (c.split_upper && c.meta_fp16) return fail("split_upper is built with fp32 metadata only");
  return true;
}

// Bytes of one (scale, zero-point / offset) pair.
inline size_t meta_bytes(const qs_config& c) { return c.meta_fp16 ? 4 : 8; }

// Record slots per (sequence, head) in the split workspace.
inline int record_slots() { return kMaxQuantSplits + kMaxTailItems; }

inline qs_layout make_layout(const qs_config& c) {
  qs_layout L{};
  const size_t lbh = (size_t)c.n_layers * c.batch * c.n_heads;
  const size_t T = (size_t)c.max_ctx, D = (size_t)c.head_dim, G = (size_t)c.group;
  L.uk_bytes = align256(lbh * T * (D / 2));
  L.uv_bytes = align256(lbh * (T / G) * D * (G / 2));
  const size_t mb = meta_bytes(c);
  L.kmeta_bytes = align256(lbh * (T / G) * D * mb);
  L.vmeta_bytes = align256(lbh * T * mb);
  L.tail_bytes = align256(lbh * 2 * G * D * 2);
  L.work_bytes = align256((size_t)c.batch * c.n_heads * record_slots() * (c.gamma_max + 1) *
                          (D + kRecPad) * sizeof(float));
  L.state_bytes = align256(((size_t)c.n_layers * c.batch * kStateInts + 1) * sizeof(int32_t));
  size_t o = 0;
  L.uk = o; o += L.uk_bytes;
  L.lk = o; o += L.uk_bytes;
  L.uv = o; o += L.uv_bytes;
  L.lv = o; o += L.uv_bytes;
  L.kmeta = o; o += L.kmeta_bytes;
  L.vmeta = o; o += L.vmeta_bytes;
  L.tail_k = o; o += L.tail_bytes;
  L.tail_v = o; o += L.tail_bytes;
  L.work = o; o += L.work_bytes;
  L.state = o; o += L.state_bytes;
  L.total = o;
  return L;
}

struct Seq {
  int32_t nq = 0;    // quantized tokens
  int32_t nt = 0;    // tail tokens
  int32_t head = 0;  // ring slot of logical tail token 0 (0 or G)
};

// Work decomposition of one attention call.
struct Plan {
  int32_t chunk_groups = 1;
  int32_t qitems[QS_MAX_BATCH] = {};
  int32_t titems[QS_MAX_BATCH] = {};
  int32_t qbase[QS_MAX_BATCH + 1] = {};
  int32_t tbase[QS_MAX_BATCH + 1] = {};
};

// Quantized work: each sequence's groups are dealt to ceil(groups / chunk_groups) workers per
// head.  The chunk length is the smallest one that keeps the call at no more than
// `target_items` (sequence, head, worker) items (so that they all run in one resident round) and
// no sequence at more than kMaxQuantSplits workers.
inline Plan make_plan(const Seq* s, int B, int H, int G, int target_items) {
  Plan p;
  long long groups = 0;
  int max_groups = 0;
  for (int b = 0; b < B; ++b) {
    int g = s[b].nq / G;
    groups += g;
    if (g > max_groups) max_groups = g;
  }
  if (target_items < 1) target_items = 1;
  long long want = (groups * H + target_items - 1) / target_items;
  int lo = (max_groups + kMaxQuantSplits - 1) / kMaxQuantSplits;
  long long cg = want > lo ? want : lo;
  if (cg < 1) cg = 1;
  auto items = [&](long long c) {
    long long n = 0;
    for (int b = 0; b < B; ++b) n += (long long)H * ((s[b].nq / G + c - 1) / c);
    return n;
  };
  while (cg < max_groups && items(cg) > target_items) ++cg;
  p.chunk_groups = (int32_t)cg;
  for (int b = 0; b < B; ++b) {
    int g = s[b].nq / G;
    p.qitems[b] = (int32_t)((g + cg - 1) / cg);
    p.titems[b] = (s[b].nt + kTailChunk - 1) / kTailChunk;
    p.qbase[b + 1] = p.qbase[b] + p.qitems[b];
    p.tbase[b + 1] = p.tbase[b] + p.titems[b];
  }
  return p;
}

// Per-(layer, sequence) counters with validate-then-apply verbs.  Every check_* returns
// QS_OK or an error with a message and leaves the state untouched.
class State {
 public:
  State() = default;
  explicit State(const qs_config& c) : cfg_(c), seq_((size_t)c.n_layers * c.batch) {}

  const qs_config& cfg() const { return cfg_; }
  Seq& at(int layer, int b) { return seq_[(size_t)layer * cfg_.batch + b]; }
  const Seq& at(int layer, int b) const { return seq_[(size_t)layer * cfg_.batch + b]; }
  int ring() const { return 2 * cfg_.group; }

  qs_status check_layer(int layer, bool allow_all, std::string* err) const {
    if ((allow_all && layer == -1) || (layer >= 0 && layer < cfg_.n_layers)) return QS_OK;
    *err = "layer out of range";
    return QS_ERR_INVALID_ARG;
  }

  // n: per-sequence counts (already defaulted to n_max by the caller).
  qs_status check_append(int layer, int n_max, const int32_t* n, std::string* err) const {
    qs_status st = check_layer(layer, false, err);
    if (st != QS_OK) return st;
    if (n_max < 0) { *err = "n_max must be >= 0"; return QS_ERR_INVALID_ARG; }
    for (int b = 0; b < cfg_.batch; ++b) {
      if (n[b] < 0 || n[b] > n_max) { *err = "n[b] must be in 0..n_max"; return QS_ERR_INVALID_ARG; }
      if (at(layer, b).nt + n[b] > ring()) {
        *err = "append would overflow the 2G-slot tail (flush first)";
        return QS_ERR_CAPACITY;
      }
    }
    return QS_OK;
  }
  void apply_append(int layer, const int32_t* n) {
    for (int b = 0; b < cfg_.batch; ++b) at(layer, b).nt += n[b];
  }

  // n: prompt tokens per sequence.  A prompt is placed after the quantized tier, so a sequence
  // that receives one must have an empty tail (its tokens would otherwise be older).
  qs_status check_prefill(int layer, int n_max, const int32_t* n, std::string* err) const {
    qs_status st = check_layer(layer, false, err);
    if (st != QS_OK) return st;
    if (n_max < 0) { *err = "n_max must be >= 0"; return QS_ERR_INVALID_ARG; }
    // grid rows: the whole groups, plus one for the rest (at most 65535)
    if (n_max / cfg_.group > 65534) { *err = "n_max / G must be <= 65534"; return QS_ERR_INVALID_ARG; }
    for (int b = 0; b < cfg_.batch; ++b) {
      if (n[b] < 0 || n[b] > n_max) { *err = "n[b] must be in 0..n_max"; return QS_ERR_INVALID_ARG; }
      if (n[b] == 0) continue;
      if (at(layer, b).nt != 0) {
        *err = "prefill needs an empty tail (flush or roll back first)";
        return QS_ERR_STATE;
      }
      if ((long long)at(layer, b).nq + (long long)(n[b] / cfg_.group) * cfg_.group > cfg_.max_ctx) {
        *err = "prefill would exceed max_ctx";
        return QS_ERR_CAPACITY;
      }
    }
    return QS_OK;
  }
  // The same counters as append(G) + flush repeated n / G times, then append(n mod G).
  void apply_prefill(int layer, const int32_t* n) {
    for (int b = 0; b < cfg_.batch; ++b) {
      Seq& s = at(layer, b);
      const int groups = n[b] / cfg_.group;
      s.nq += groups * cfg_.group;
      if (groups & 1) s.head ^= cfg_.group;
      s.nt += n[b] % cfg_.group;
    }
  }

  qs_status check_rollback(int layer, const int32_t* drop, std::string* err) const {
    qs_status st = check_layer(layer, true, err);
    if (st != QS_OK || !drop) return st;
    int l0 = layer < 0 ? 0 : layer, l1 = layer < 0 ? cfg_.n_layers : layer + 1;
    for (int l = l0; l < l1; ++l)
      for (int b = 0; b < cfg_.batch; ++b) {
        if (drop[b] < 0) { *err = "n_drop[b] must be >= 0"; return QS_ERR_INVALID_ARG; }
        if (drop[b] > at(l, b).nt) {
          *err = "rollback past the tail: quantized tokens are never rolled back";
          return QS_ERR_STATE;
        }
      }
    return QS_OK;
  }
  void apply_rollback(int layer, const int32_t* drop) {
    if (!drop) return;
    int l0 = layer < 0 ? 0 : layer, l1 = layer < 0 ? cfg_.n_layers : layer + 1;
    for (int l = l0; l < l1; ++l)
      for (int b = 0; b < cfg_.batch; ++b) at(l, b).nt -= drop[b];
  }

  int flush_threshold(int min_tail) const { return min_tail > cfg_.group ? min_tail : cfg_.group; }
  bool selected(int layer, int b, int min_tail) const {
    return at(layer, b).nt >= flush_threshold(min_tail);
  }
  qs_status check_flush(int layer, int min_tail, std::string* err) const {
    qs_status st = check_layer(layer, true, err);
    if (st != QS_OK) return st;
    if (min_tail > ring()) { *err = "min_tail must be <= 2G"; return QS_ERR_INVALID_ARG; }
    int l0 = layer < 0 ? 0 : layer, l1 = layer < 0 ? cfg_.n_layers : layer + 1;
    for (int l = l0; l < l1; ++l)
      for (int b = 0; b < cfg_.batch; ++b)
        if (selected(l, b, min_tail) && at(l, b).nq + cfg_.group > cfg_.max_ctx) {
          *err = "flush would exceed max_ctx";
          return QS_ERR_CAPACITY;
        }
    return QS_OK;
  }
  void apply_flush_one(int layer, int b) {
    Seq& s = at(layer, b);
    s.nq += cfg_.group;
    s.nt -= cfg_.group;
    s.head ^= cfg_.group;
  }

  qs_status check_attend(int layer, int m, bool draft, std::string* err) const {
    qs_status st = check_layer(layer, false, err);
    if (st != QS_OK) return st;
    if (!draft && (m < 1 || m > cfg_.gamma_max + 1)) {
      *err = "m must be in 1..gamma_max+1";
      return QS_ERR_INVALID_ARG;
    }
    for (int b = 0; b < cfg_.batch; ++b) {
      const Seq& s = at(layer, b);
      if (s.nq + s.nt == 0) { *err = "attention over a sequence that holds no token"; return QS_ERR_STATE; }
      if (!draft && m > s.nt) { *err = "verify needs m <= nt (the m queries are tail tokens)"; return QS_ERR_STATE; }
    }
    return QS_OK;
  }

 private:
  qs_config cfg_{};
  std::vector<Seq> seq_;
};

}  // namespace qs
