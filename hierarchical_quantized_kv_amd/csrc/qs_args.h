// qs_args.h -- plain-old-data kernel arguments shared by the host library and the HIP kernels.
// Everything a kernel needs about the per-sequence bookkeeping is passed by value, so no call
// copies host data to the device and no host buffer has to outlive its launch -- except in
// device mode, where the kernels read the counters from the arena's state section (dstate) and
// the by-value copies are unused.
#pragma once

#include <stdint.h>

#include "../../include/quantspec.h"

namespace qs {

constexpr int kGroup = 128;           // G: tokens per quantization group (keys) / ring half
constexpr int kTailChunk = 64;        // tail tokens handled by one tail work item
constexpr int kMaxTailItems = 2 * kGroup / kTailChunk;
constexpr int kMaxQuantSplits = 256;  // quantized work items per (sequence, head), at most
constexpr int kRecPad = 4;            // partial record = [max, sum, pad, pad, o[D]]
constexpr int kStateInts = 4;         // device state per (layer, sequence): nq, nt, head, pad

// Device mode: counter changes of appends and rollbacks not yet written to the state section.
// Every kernel that reads nt applies them in order (with the same checks as the host verbs, a
// failing operation being skipped); the next attention call's combine kernel, or the state
// kernel of a flush or commit, writes the result back -- after every reader of the old value
// has finished.  So appends and rollbacks launch no kernel of their own for the counters.
constexpr int kMaxPending = 4;
struct PendingOp {
  int32_t kind;        // 0: append n tokens; 1: roll back n - sub[b] tokens
  int32_t n;
  const int32_t* sub;  // rollback: device int32 [B] (or null)
};
struct Pending {
  int32_t count;
  PendingOp op[kMaxPending];
};

// Bits of the device-mode error word (the int32 after the last (layer, sequence) entry).
enum : int32_t {
  kDevErrAppend = 1,    // an append would have overflowed the 2G-slot tail (nothing written)
  kDevErrRollback = 2,  // a rollback count was negative or past the tail (state unchanged)
  kDevErrFlush = 4,     // a selected flush would have exceeded max_ctx (nothing written)
  kDevErrAttend = 8,    // attention over an empty sequence, or verify with m > nt
};

// One attention call (draft or verify) on one layer: the fields that do not depend on the batch.
struct AttnHeader {
  const uint8_t* uk;     // layer base of each section
  const uint8_t* lk;
  const uint8_t* uv;
  const uint8_t* lv;
  const uint8_t* kmeta;  // (scale, zero-point) fp32 pairs, or (scale, offset) fp16 pairs
  const uint8_t* vmeta;
  const uint16_t* tail_k;
  const uint16_t* tail_v;
  const uint16_t* q;     // draft [B][H][D], verify [B][m][H][D]
  float* out;            // same shape as q, fp32
  float* work;           // partial records [B][H][S][m][D + kRecPad]
  int32_t B, H, T, NG;   // batch, heads, token capacity, groups per sequence
  int32_t m;             // queries per (sequence, head)
  int32_t S;             // record slots per (sequence, head) = kMaxQuantSplits + kMaxTailItems
  int32_t chunk_groups;  // quantized groups per worker, at most (sizes the worker count)
  int32_t n_qitems_total, n_titems_total;
  float qscale;          // sm_scale * log2(e): scores are kept in the base-2 domain
  float draft_offset;    // 8 or 0 (draft only)
  int32_t meta16;        // fp16 metadata (selects the kernel instantiation)
};

// Per-sequence bookkeeping for at most NB sequences.  The kernels are instantiated for a few
// NB (1, 8, QS_MAX_BATCH) so that a small batch passes a small argument block: every launch
// copies its argument block, and at NB = QS_MAX_BATCH (about 1.7 KB) that copy costs more
// than a microsecond of launch latency.
// Variants of an attention call (a template parameter of the kernels: each its own
// instantiation, so the plain one carries none of the others' fields or code).
enum : int {
  kModeHost = 0,    // counters by value
  kModeDev = 1,     // counters from the state section (device mode)
  kModeAppend = 2,  // counters by value, and the call first appends tokens to the tail
  kModeGqa = 3,     // counters by value; gq query heads share each cached (key/value) head
};

// The grouped-query draft runs the MFMA item's paired form (hi and lo parts of a query in the
// columns j and j + 8 of one B operand) when its query columns fit in half an MFMA tile.
constexpr int kPairMaxQueries = 8;
constexpr bool gqa_paired(bool draft, int m) { return draft && m <= kPairMaxQueries; }

// Layout of the upper planes that an attention kernel reads (a template parameter too):
//   kFmtNibble  the upper nibble C_U as one 4-bit plane per stream (uk, uv);
//   kFmtSplit4  split-upper layout: C_U = 4 C_T + C_M stored as a 2-bit top plane (first half of
//               each (layer, sequence, head) stripe of uk / uv) and a 2-bit middle plane (second
//               half), read back into nibbles by the 4-bit draft and by verify;
//   kFmtSplit2  split-upper layout, the 2-bit draft: only the top plane is read.
enum : int { kFmtNibble = 0, kFmtSplit4 = 1, kFmtSplit2 = 2 };

template <int NB, int MODE = kModeHost>
struct AttnArgsN : AttnHeader {
  static constexpr int kMode = kModeHost;
  int32_t nq[NB];                // quantized tokens per sequence
  int32_t nt[NB];                // tail tokens per sequence
  int32_t head[NB];              // ring slot of logical tail token 0
  int32_t qitem_base[NB + 1];    // prefix sum over b of quantized workers
  int32_t titem_base[NB + 1];    // prefix sum over b of tail items
};
using AttnArgs = AttnArgsN<QS_MAX_BATCH>;

// Device mode: the counters come from the state section instead of nq / nt / head (a separate
// instantiation of the kernels, so the host-mode ones carry none of this).
struct AttnDev {
  const int32_t* dstate; // this layer's [B][kStateInts] counters
  int32_t* wstate;       // where the combine kernel commits the pending operations (= dstate)
  int32_t* derr;         // the error word
  int32_t min_nt;        // tail tokens the call needs (verify: m; draft: 0)
  Pending pend;          // this layer's pending operations
};
template <int NB>
struct AttnArgsN<NB, kModeDev> : AttnArgsN<NB, kModeHost> {
  static constexpr int kMode = kModeDev;
  AttnDev dev;
};
using AttnDevArgs = AttnArgsN<QS_MAX_BATCH, kModeDev>;

// Fused append: before attending, the call appends an[b] tokens of ak / av [B][an_max][H][D] to
// sequence b's tail (nt[] already counts them).  The tail item whose chunk holds a new token's
// ring slot reads the token from ak / av, writes it to the ring and attends over it in the same
// pass, so no separate append kernel runs.
template <int NB>
struct AttnArgsN<NB, kModeAppend> : AttnArgsN<NB, kModeHost> {
  static constexpr int kMode = kModeAppend;
  const uint16_t* ak;
  const uint16_t* av;
  uint16_t* wtail_k;     // the ring again, writable (= tail_k / tail_v)
  uint16_t* wtail_v;
  int32_t an_max;
  int32_t an[NB];
};
using AttnAppArgs = AttnArgsN<QS_MAX_BATCH, kModeAppend>;

// Grouped queries: query head h * gq + r (r < gq) reads cached head h.  The m query columns of a
// (sequence, cached head) are c = i * gq + r for query token i < mt (m = mt * gq <= 16); q and
// out are [B][mt][hq][D] with hq = H * gq.  Both passes run the MFMA item; the draft one reads
// only the upper planes.
template <int NB>
struct AttnArgsN<NB, kModeGqa> : AttnArgsN<NB, kModeHost> {
  static constexpr int kMode = kModeGqa;
  int32_t gq, mt, hq;
};
using AttnGqaArgs = AttnArgsN<QS_MAX_BATCH, kModeGqa>;

struct AppendHeader {
  const uint16_t* k;     // [B][n_max][H][D]
  const uint16_t* v;
  uint16_t* tail_k;      // layer base [B][H][2G][D]
  uint16_t* tail_v;
  int32_t B, H, n_max;
  int32_t n_rows;        // tokens per sequence the grid covers (n_max, or a prefill's longest rest)
  const int32_t* dstate; // device mode: this layer's [B][kStateInts] counters (start = nt); else null
  Pending pend;          // device mode: this layer's pending operations, before this append
};

template <int NB>
struct AppendArgsN : AppendHeader {
  int32_t n[NB];      // tokens appended per sequence
  int32_t start[NB];  // logical position nt before the append
  int32_t head[NB];
  int32_t src0[NB];   // first source token of the sequence in k / v (0 but for a prefill's rest)
};
using AppendArgs = AppendArgsN<QS_MAX_BATCH>;

// Batch bucket of the kernel instantiation that serves a batch of B sequences.
inline int batch_bucket(int B) { return B <= 1 ? 1 : (B <= 8 ? 8 : QS_MAX_BATCH); }

// Bulk prefill of one layer: whole G-token groups of a prompt quantized straight from the
// caller's K / V (the rest of each prompt goes to the tail through the append kernel).
struct PrefillArgs {
  uint8_t* uk;           // arena section bases (all layers)
  uint8_t* lk;
  uint8_t* uv;
  uint8_t* lv;
  uint8_t* kmeta;        // fp32 (scale, zero-point) or, with meta16, fp16 (scale, offset)
  uint8_t* vmeta;
  int32_t meta16;
  int32_t split;         // split-upper layout: uk / uv hold the top and middle 2-bit planes
  const uint16_t* k;     // prompt [B][n_max][H][D]
  const uint16_t* v;
  int32_t B, H, T, NG;
  int32_t layer, n_max;
  int32_t groups[QS_MAX_BATCH];  // whole groups of each sequence's prompt
  int32_t group0[QS_MAX_BATCH];  // quantized-tier group index of the first of them (nq / G)
  // the rest of each prompt (n mod G tokens after its whole groups) goes to the ring in the same
  // launch, by the workgroups of row rest_row (-1: no rest anywhere)
  uint16_t* tail_k;              // this layer's ring [B][H][2G][D]
  uint16_t* tail_v;
  int32_t rest_row;
  int32_t rest[QS_MAX_BATCH];       // n mod G of each prompt
  int32_t rest_slot[QS_MAX_BATCH];  // ring slot of its first rest token
};

struct FlushArgs {
  uint8_t* uk;           // arena section bases (all layers)
  uint8_t* lk;
  uint8_t* uv;
  uint8_t* lv;
  uint8_t* kmeta;        // fp32 (scale, zero-point) or, with meta16, fp16 (scale, offset)
  uint8_t* vmeta;
  int32_t meta16;
  int32_t split;         // split-upper layout: uk / uv hold the top and middle 2-bit planes
  const uint16_t* tail_k;
  const uint16_t* tail_v;
  int32_t B, H, T, NG;
  int32_t layer0;              // first layer of the launch; blockIdx.z adds to it
  int32_t n_sel;               // selected sequences
  int32_t b[QS_MAX_BATCH];     // selected sequence ids
  int32_t group[QS_MAX_BATCH]; // destination group index nq / G
  int32_t head[QS_MAX_BATCH];  // ring slot of the oldest tail token (0 or G)
  // device mode: the counters of all layers [L][B][kStateInts]; every sequence is in b[], and a
  // block quantizes only if nt >= thr and nq + G <= T (group and head come from the counters)
  const int32_t* dstate;
  int32_t thr;
  Pending pend;          // pending operations of every layer of the launch (the same list)
};

// Device-mode commit of the pending operations of layers l0 .. l0+nl-1 (the same list for all),
// then, for op 1, the flush's counter update; one thread per (layer, sequence).
struct StateArgs {
  int32_t* state;        // [L][B][kStateInts]
  int32_t* err;          // error word
  int32_t op;            // 0 commit only, 1 commit then flush (nt >= thr)
  int32_t l0, nl, B;
  int32_t thr, G, T;
  Pending pend;
};

}  // namespace qs
