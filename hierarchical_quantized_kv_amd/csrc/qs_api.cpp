// qs_api.cpp -- the C ABI of include/quantspec.h: validation, bookkeeping and kernel launches.
//
// Every verb validates all of its arguments against the host-side State first, then enqueues
// its kernels on the caller's stream, and only then updates the State.  No verb synchronizes
// with the device or copies host data to it: per-sequence counters travel as kernel arguments.
// In device mode (qs_state_to_device .. qs_state_from_device) the counters live in the arena's
// state section instead.  Appends and rollbacks are recorded as pending operations of their
// layer, passed by value to every later kernel that reads the counters and committed by the
// next attention call (its combine kernel), flush or commit; so the _dev verbs launch the same
// kernels as the host verbs (plus one small kernel per flush) and a sequence of them can be
// captured in a graph and replayed, provided it starts and ends with nothing pending.
#include <hip/hip_runtime.h>

#include <math.h>
#include <string.h>

#include <new>
#include <string>
#include <vector>

#include "../../include/quantspec.h"
#include "qs_state.h"

namespace qs {
hipError_t launch_append(const AppendArgs& a, int D, hipStream_t st);
hipError_t launch_flush(const FlushArgs& a, int D, int n_layers, hipStream_t st);
hipError_t launch_prefill(const PrefillArgs& a, int D, int max_groups, hipStream_t st);
hipError_t launch_attention(const AttnArgs& a, int D, bool draft, hipStream_t st);
hipError_t launch_attention_dev(const AttnDevArgs& a, int D, bool draft, hipStream_t st);
hipError_t launch_attention_app(const AttnAppArgs& a, int D, bool draft, hipStream_t st);
hipError_t launch_attention_gqa(const AttnGqaArgs& a, int D, bool draft, hipStream_t st);
hipError_t launch_attention_split(const AttnArgs& a, int D, bool draft, int fmt, hipStream_t st);
hipError_t launch_attention_app_split(const AttnAppArgs& a, int D, bool draft, hipStream_t st);
hipError_t launch_state(const StateArgs& a, hipStream_t st);
int attention_slots(int D, bool draft, int B, int mode, bool meta16, int fmt, bool pair = false);
}  // namespace qs

struct qs_cache {
  qs_config cfg;
  qs_layout lay;
  uint8_t* arena;
  qs::State st;
  std::string err;
  bool dev = false;  // device mode: the counters are in the state section, not in st
  std::vector<qs::Pending> pend;  // device mode: per layer, operations not yet committed
};

namespace {

// Work items per attention call: one resident round of waves, i.e. the pass kernel's slots on the
// device (compute units x resident one-wave workgroups) minus the tail items; 2048 if unknown.
constexpr int kFallbackSlots = 2048;

qs_status fail(qs_cache* c, qs_status s, const std::string& m) {
  if (c) c->err = m;
  return s;
}

qs_status device_fail(qs_cache* c, hipError_t e, const char* what) {
  return fail(c, QS_ERR_DEVICE, std::string(what) + ": " + hipGetErrorString(e));
}

size_t layer_off(const qs_cache* c, size_t per_lbh_bytes, int layer) {
  return (size_t)layer * c->cfg.batch * c->cfg.n_heads * per_lbh_bytes;
}

const char* const kInDeviceMode = "the counters are on the device (qs_state_from_device first)";
const char* const kNotSplit = "not available with split_upper (host-mode and fused calls only)";
const char* const kInHostMode = "not in device mode (qs_state_to_device first)";

int32_t* dev_state(const qs_cache* c) { return reinterpret_cast<int32_t*>(c->arena + c->lay.state); }
int32_t* dev_error(const qs_cache* c) {
  return dev_state(c) + (size_t)c->cfg.n_layers * c->cfg.batch * qs::kStateInts;
}

}  // namespace

extern "C" {

size_t qs_arena_bytes(const qs_config* cfg) {
  if (!cfg || !qs::config_ok(*cfg, nullptr)) return 0;
  return qs::make_layout(*cfg).total;
}

qs_status qs_arena_layout(const qs_config* cfg, qs_layout* out) {
  if (!cfg || !out || !qs::config_ok(*cfg, nullptr)) return QS_ERR_INVALID_ARG;
  *out = qs::make_layout(*cfg);
  return QS_OK;
}

qs_status qs_cache_create(const qs_config* cfg, void* d_arena, size_t arena_bytes, qs_cache** out) {
  if (!cfg || !out) return QS_ERR_INVALID_ARG;
  *out = nullptr;
  if (!qs::config_ok(*cfg, nullptr)) return QS_ERR_INVALID_ARG;
  const qs_layout lay = qs::make_layout(*cfg);
  if (!d_arena || ((uintptr_t)d_arena & 255) || arena_bytes < lay.total) return QS_ERR_BUFFER;
  qs_cache* c = new (std::nothrow) qs_cache();
  if (!c) return QS_ERR_DEVICE;
  c->cfg = *cfg;
  c->lay = lay;
  c->arena = static_cast<uint8_t*>(d_arena);
  c->st = qs::State(*cfg);
  *out = c;
  return QS_OK;
}

qs_status qs_cache_destroy(qs_cache* cache) {
  delete cache;
  return QS_OK;
}

qs_status qs_append(qs_cache* c, int32_t layer, const void* d_k, const void* d_v, int32_t n_max,
                    const int32_t* h_n, void* stream) {
  if (!c) return QS_ERR_INVALID_ARG;
  if (c->dev) return fail(c, QS_ERR_STATE, kInDeviceMode);
  if (!d_k || !d_v) return fail(c, QS_ERR_INVALID_ARG, "null k or v");
  const qs_config& cf = c->cfg;
  int32_t n[QS_MAX_BATCH];
  for (int b = 0; b < cf.batch; ++b) n[b] = h_n ? h_n[b] : n_max;
  std::string err;
  qs_status s = c->st.check_append(layer, n_max, n, &err);
  if (s != QS_OK) return fail(c, s, err);
  qs::AppendArgs a{};
  a.k = static_cast<const uint16_t*>(d_k);
  a.v = static_cast<const uint16_t*>(d_v);
  const size_t tail_lbh = (size_t)2 * cf.group * cf.head_dim * 2;
  a.tail_k = reinterpret_cast<uint16_t*>(c->arena + c->lay.tail_k + layer_off(c, tail_lbh, layer));
  a.tail_v = reinterpret_cast<uint16_t*>(c->arena + c->lay.tail_v + layer_off(c, tail_lbh, layer));
  a.B = cf.batch;
  a.H = cf.n_heads;
  a.n_max = n_max;
  a.n_rows = n_max;
  int total = 0;
  for (int b = 0; b < cf.batch; ++b) {
    a.n[b] = n[b];
    a.start[b] = c->st.at(layer, b).nt;
    a.head[b] = c->st.at(layer, b).head;
    total += n[b];
  }
  if (total > 0) {
    hipError_t e = qs::launch_append(a, cf.head_dim, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return device_fail(c, e, "append launch");
  }
  c->st.apply_append(layer, n);
  c->err.clear();
  return QS_OK;
}

qs_status qs_prefill(qs_cache* c, int32_t layer, const void* d_k, const void* d_v, int32_t n_max,
                     const int32_t* h_n, void* stream) {
  if (!c) return QS_ERR_INVALID_ARG;
  if (c->dev) return fail(c, QS_ERR_STATE, kInDeviceMode);
  if (!d_k || !d_v) return fail(c, QS_ERR_INVALID_ARG, "null k or v");
  const qs_config& cf = c->cfg;
  int32_t n[QS_MAX_BATCH];
  for (int b = 0; b < cf.batch; ++b) n[b] = h_n ? h_n[b] : n_max;
  std::string err;
  qs_status s = c->st.check_prefill(layer, n_max, n, &err);
  if (s != QS_OK) return fail(c, s, err);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  // whole groups: quantized straight from the prompt
  qs::PrefillArgs p{};
  p.uk = c->arena + c->lay.uk;
  p.lk = c->arena + c->lay.lk;
  p.uv = c->arena + c->lay.uv;
  p.lv = c->arena + c->lay.lv;
  p.kmeta = c->arena + c->lay.kmeta;
  p.vmeta = c->arena + c->lay.vmeta;
  p.meta16 = cf.meta_fp16;
  p.split = cf.split_upper;
  p.k = static_cast<const uint16_t*>(d_k);
  p.v = static_cast<const uint16_t*>(d_v);
  p.B = cf.batch;
  p.H = cf.n_heads;
  p.T = cf.max_ctx;
  p.NG = cf.max_ctx / cf.group;
  p.layer = layer;
  p.n_max = n_max;
  // the rest of each prompt goes into the ring in the same launch, where the equivalent append /
  // flush sequence leaves it (the ring head toggles once per quantized group; the tail was empty)
  const size_t tail_lbh = (size_t)2 * cf.group * cf.head_dim * 2;
  p.tail_k = reinterpret_cast<uint16_t*>(c->arena + c->lay.tail_k + layer_off(c, tail_lbh, layer));
  p.tail_v = reinterpret_cast<uint16_t*>(c->arena + c->lay.tail_v + layer_off(c, tail_lbh, layer));
  int max_groups = 0, rest = 0;
  for (int b = 0; b < cf.batch; ++b) {
    const qs::Seq& q = c->st.at(layer, b);
    p.groups[b] = n[b] / cf.group;
    p.group0[b] = q.nq / cf.group;
    if (p.groups[b] > max_groups) max_groups = p.groups[b];
    p.rest[b] = n[b] % cf.group;
    const int head = (p.groups[b] & 1) ? (q.head ^ cf.group) : q.head;
    p.rest_slot[b] = (head + q.nt) % (2 * cf.group);  // nt is 0 whenever n[b] > 0
    rest += p.rest[b];
  }
  p.rest_row = rest > 0 ? max_groups : -1;
  hipError_t e = qs::launch_prefill(p, cf.head_dim, max_groups, st);
  if (e != hipSuccess) return device_fail(c, e, "prefill launch");
  c->st.apply_prefill(layer, n);
  c->err.clear();
  return QS_OK;
}

qs_status qs_rollback(qs_cache* c, int32_t layer, const int32_t* h_n_drop) {
  if (!c) return QS_ERR_INVALID_ARG;
  if (c->dev) return fail(c, QS_ERR_STATE, kInDeviceMode);
  std::string err;
  qs_status s = c->st.check_rollback(layer, h_n_drop, &err);
  if (s != QS_OK) return fail(c, s, err);
  c->st.apply_rollback(layer, h_n_drop);
  c->err.clear();
  return QS_OK;
}

qs_status qs_flush(qs_cache* c, int32_t layer, int32_t min_tail, void* stream, int32_t* h_flushed) {
  if (!c) return QS_ERR_INVALID_ARG;
  if (c->dev) return fail(c, QS_ERR_STATE, kInDeviceMode);
  std::string err;
  qs_status s = c->st.check_flush(layer, min_tail, &err);
  if (s != QS_OK) return fail(c, s, err);
  const qs_config& cf = c->cfg;
  const int l0 = layer < 0 ? 0 : layer, l1 = layer < 0 ? cf.n_layers : layer + 1;
  qs::FlushArgs a{};
  a.uk = c->arena + c->lay.uk;
  a.lk = c->arena + c->lay.lk;
  a.uv = c->arena + c->lay.uv;
  a.lv = c->arena + c->lay.lv;
  a.kmeta = c->arena + c->lay.kmeta;
  a.vmeta = c->arena + c->lay.vmeta;
  a.meta16 = cf.meta_fp16;
  a.split = cf.split_upper;
  a.tail_k = reinterpret_cast<const uint16_t*>(c->arena + c->lay.tail_k);
  a.tail_v = reinterpret_cast<const uint16_t*>(c->arena + c->lay.tail_v);
  a.B = cf.batch;
  a.H = cf.n_heads;
  a.T = cf.max_ctx;
  a.NG = cf.max_ctx / cf.group;
  // Consecutive layers whose selected sequences share (group index, ring head) go in one launch.
  auto same = [&](int la, int lb) {
    for (int b = 0; b < cf.batch; ++b) {
      const bool sa = c->st.selected(la, b, min_tail), sb = c->st.selected(lb, b, min_tail);
      if (sa != sb) return false;
      if (sa && (c->st.at(la, b).nq != c->st.at(lb, b).nq || c->st.at(la, b).head != c->st.at(lb, b).head))
        return false;
    }
    return true;
  };
  int32_t last_sel[QS_MAX_BATCH];
  for (int b = 0; b < cf.batch; ++b) last_sel[b] = c->st.selected(l1 - 1, b, min_tail) ? 1 : 0;
  int run0 = l0;
  while (run0 < l1) {
    int run1 = run0 + 1;
    while (run1 < l1 && same(run0, run1)) ++run1;
    a.layer0 = run0;
    a.n_sel = 0;
    for (int b = 0; b < cf.batch; ++b)
      if (c->st.selected(run0, b, min_tail)) {
        a.b[a.n_sel] = b;
        a.group[a.n_sel] = c->st.at(run0, b).nq / cf.group;
        a.head[a.n_sel] = c->st.at(run0, b).head;
        ++a.n_sel;
      }
    if (a.n_sel > 0) {
      hipError_t e = qs::launch_flush(a, cf.head_dim, run1 - run0, static_cast<hipStream_t>(stream));
      if (e != hipSuccess) return device_fail(c, e, "flush launch");
      for (int l = run0; l < run1; ++l)
        for (int k = 0; k < a.n_sel; ++k) c->st.apply_flush_one(l, a.b[k]);
    }
    run0 = run1;
  }
  if (h_flushed)
    for (int b = 0; b < cf.batch; ++b) h_flushed[b] = last_sel[b];
  c->err.clear();
  return QS_OK;
}

// Argument block of one attention call of `layer` over the work plan p.
static void attn_args(const qs_cache* c, int32_t layer, const void* d_q, int32_t m, float sm_scale,
                      float* d_out, const qs::Plan& p, qs::AttnArgs& a) {
  const qs_config& cf = c->cfg;
  const int D = cf.head_dim;
  const size_t T = cf.max_ctx, G = cf.group, NG = T / G;
  a.uk = c->arena + c->lay.uk + layer_off(c, T * (D / 2), layer);
  a.lk = c->arena + c->lay.lk + layer_off(c, T * (D / 2), layer);
  a.uv = c->arena + c->lay.uv + layer_off(c, NG * D * (G / 2), layer);
  a.lv = c->arena + c->lay.lv + layer_off(c, NG * D * (G / 2), layer);
  const size_t mb = qs::meta_bytes(cf);
  a.kmeta = c->arena + c->lay.kmeta + layer_off(c, NG * D * mb, layer);
  a.vmeta = c->arena + c->lay.vmeta + layer_off(c, T * mb, layer);
  a.tail_k = reinterpret_cast<const uint16_t*>(c->arena + c->lay.tail_k + layer_off(c, 2 * G * D * 2, layer));
  a.tail_v = reinterpret_cast<const uint16_t*>(c->arena + c->lay.tail_v + layer_off(c, 2 * G * D * 2, layer));
  a.q = static_cast<const uint16_t*>(d_q);
  a.out = d_out;
  a.work = reinterpret_cast<float*>(c->arena + c->lay.work);
  a.B = cf.batch;
  a.H = cf.n_heads;
  a.T = cf.max_ctx;
  a.NG = (int32_t)NG;
  a.m = m;
  a.S = qs::record_slots();
  a.chunk_groups = p.chunk_groups;
  a.n_qitems_total = p.qbase[cf.batch];
  a.n_titems_total = p.tbase[cf.batch];
  a.qscale = sm_scale * 1.4426950408889634f;
  a.draft_offset = (float)cf.draft_offset;
  a.meta16 = cf.meta_fp16;
  for (int b = 0; b <= cf.batch; ++b) {
    a.qitem_base[b] = p.qbase[b];
    a.titem_base[b] = p.tbase[b];
  }
}

// Work plan for the sequences `seqs`: quantized workers sized to one resident round of the pass
// kernel (pair: the grouped-query draft's paired form), next to the tail items.
static qs::Plan attn_plan(const qs_cache* c, const qs::Seq* seqs, bool draft, int mode,
                          int fmt = qs::kFmtNibble, bool pair = false) {
  const qs_config& cf = c->cfg;
  int slots = qs::attention_slots(cf.head_dim, draft, cf.batch, mode, cf.meta_fp16 != 0, fmt, pair);
  if (slots <= 0) slots = kFallbackSlots;
  int tail_items = 0;
  for (int b = 0; b < cf.batch; ++b)
    tail_items += cf.n_heads * ((seqs[b].nt + qs::kTailChunk - 1) / qs::kTailChunk);
  const int target = slots - tail_items > slots / 2 ? slots - tail_items : slots / 2;
  return qs::make_plan(seqs, cf.batch, cf.n_heads, cf.group, target);
}

// bits: the draft's top code bits (4, or 2 with the split-upper layout); verify reads all 8.
static qs_status attend(qs_cache* c, int32_t layer, const void* d_q, int32_t m, float sm_scale,
                        float* d_out, void* stream, bool draft, int bits = 4) {
  if (!c) return QS_ERR_INVALID_ARG;
  if (c->dev) return fail(c, QS_ERR_STATE, kInDeviceMode);
  if (!d_q || !d_out) return fail(c, QS_ERR_INVALID_ARG, "null q or out");
  if (!isfinite(sm_scale)) return fail(c, QS_ERR_INVALID_ARG, "sm_scale must be finite");
  const qs_config& cf = c->cfg;
  if (bits != 4 && bits != 2) return fail(c, QS_ERR_INVALID_ARG, "bits must be 2 or 4");
  if (bits == 2 && !cf.split_upper)
    return fail(c, QS_ERR_INVALID_ARG, "a 2-bit draft needs the split-upper layout (split_upper = 1)");
  std::string err;
  qs_status s = c->st.check_attend(layer, m, draft, &err);
  if (s != QS_OK) return fail(c, s, err);
  const int fmt = !cf.split_upper ? qs::kFmtNibble : (bits == 2 ? qs::kFmtSplit2 : qs::kFmtSplit4);
  qs::Seq seqs[QS_MAX_BATCH];
  for (int b = 0; b < cf.batch; ++b) seqs[b] = c->st.at(layer, b);
  const qs::Plan p = attn_plan(c, seqs, draft, qs::kModeHost, fmt);
  qs::AttnArgs a{};
  attn_args(c, layer, d_q, m, sm_scale, d_out, p, a);
  for (int b = 0; b < cf.batch; ++b) {
    a.nq[b] = seqs[b].nq;
    a.nt[b] = seqs[b].nt;
    a.head[b] = seqs[b].head;
  }
  hipError_t e = fmt == qs::kFmtNibble
                     ? qs::launch_attention(a, cf.head_dim, draft, static_cast<hipStream_t>(stream))
                     : qs::launch_attention_split(a, cf.head_dim, draft, fmt,
                                                  static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_fail(c, e, draft ? "draft launch" : "verify launch");
  c->err.clear();
  return QS_OK;
}

// Grouped queries: g query heads per cached head, mt query tokens (1 for the draft); the m =
// mt * g query columns of a (sequence, cached head) share its split workspace, so m <= gamma_max
// + 1.
static qs_status attend_gqa(qs_cache* c, int32_t layer, const void* d_q, int32_t mt, int32_t g,
                            float sm_scale, float* d_out, void* stream, bool draft) {
  if (!c) return QS_ERR_INVALID_ARG;
  if (c->dev) return fail(c, QS_ERR_STATE, kInDeviceMode);
  if (!d_q || !d_out) return fail(c, QS_ERR_INVALID_ARG, "null q or out");
  if (!isfinite(sm_scale)) return fail(c, QS_ERR_INVALID_ARG, "sm_scale must be finite");
  const qs_config& cf = c->cfg;
  if (cf.split_upper) return fail(c, QS_ERR_INVALID_ARG, kNotSplit);
  if (g < 1 || g > QS_MAX_QUERIES) return fail(c, QS_ERR_INVALID_ARG, "g must be in 1..16");
  if (!draft && (mt < 1 || mt > cf.gamma_max + 1))
    return fail(c, QS_ERR_INVALID_ARG, "m must be in 1..gamma_max+1");
  if ((long long)mt * g > cf.gamma_max + 1)
    return fail(c, QS_ERR_INVALID_ARG, "m * g must be <= gamma_max + 1 (query columns per head)");
  std::string err;
  qs_status s = c->st.check_attend(layer, mt, draft, &err);
  if (s != QS_OK) return fail(c, s, err);
  qs::Seq seqs[QS_MAX_BATCH];
  for (int b = 0; b < cf.batch; ++b) seqs[b] = c->st.at(layer, b);
  const qs::Plan p = attn_plan(c, seqs, draft, qs::kModeGqa, qs::kFmtNibble, qs::gqa_paired(draft, mt * g));
  qs::AttnGqaArgs a{};
  attn_args(c, layer, d_q, mt * g, sm_scale, d_out, p, a);
  for (int b = 0; b < cf.batch; ++b) {
    a.nq[b] = seqs[b].nq;
    a.nt[b] = seqs[b].nt;
    a.head[b] = seqs[b].head;
  }
  a.gq = g;
  a.mt = mt;
  a.hq = cf.n_heads * g;
  hipError_t e = qs::launch_attention_gqa(a, cf.head_dim, draft, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_fail(c, e, draft ? "draft launch" : "verify launch");
  c->err.clear();
  return QS_OK;
}

// Append n[b] tokens of d_k / d_v [B][n_max][H][D], then attend: one launch pair, the tail
// items writing the new tokens to the ring as they read them.  Validation is that of the two
// verbs in sequence, all before anything changes.
static qs_status append_attend(qs_cache* c, int32_t layer, const void* d_k, const void* d_v,
                               int32_t n_max, const int32_t* h_n, const void* d_q, int32_t m,
                               float sm_scale, float* d_out, void* stream, bool draft) {
  if (!c) return QS_ERR_INVALID_ARG;
  if (c->dev) return fail(c, QS_ERR_STATE, kInDeviceMode);
  if (!d_k || !d_v) return fail(c, QS_ERR_INVALID_ARG, "null k or v");
  if (!d_q || !d_out) return fail(c, QS_ERR_INVALID_ARG, "null q or out");
  if (!isfinite(sm_scale)) return fail(c, QS_ERR_INVALID_ARG, "sm_scale must be finite");
  const qs_config& cf = c->cfg;
  int32_t n[QS_MAX_BATCH];
  for (int b = 0; b < cf.batch; ++b) n[b] = h_n ? h_n[b] : n_max;
  std::string err;
  qs_status s = c->st.check_append(layer, n_max, n, &err);
  if (s != QS_OK) return fail(c, s, err);
  qs::Seq seqs[QS_MAX_BATCH];
  for (int b = 0; b < cf.batch; ++b) {
    seqs[b] = c->st.at(layer, b);
    seqs[b].nt += n[b];
  }
  if (!draft && (m < 1 || m > cf.gamma_max + 1))
    return fail(c, QS_ERR_INVALID_ARG, "m must be in 1..gamma_max+1");
  for (int b = 0; b < cf.batch; ++b) {
    if (seqs[b].nq + seqs[b].nt == 0) return fail(c, QS_ERR_STATE, "attention over a sequence that holds no token");
    if (!draft && m > seqs[b].nt) return fail(c, QS_ERR_STATE, "verify needs m <= nt (the m queries are tail tokens)");
  }
  const int fmt = cf.split_upper ? qs::kFmtSplit4 : qs::kFmtNibble;
  const qs::Plan p = attn_plan(c, seqs, draft, qs::kModeAppend, fmt);
  qs::AttnAppArgs a{};
  attn_args(c, layer, d_q, m, sm_scale, d_out, p, a);
  for (int b = 0; b < cf.batch; ++b) {
    a.nq[b] = seqs[b].nq;
    a.nt[b] = seqs[b].nt;
    a.head[b] = seqs[b].head;
    a.an[b] = n[b];
  }
  a.ak = static_cast<const uint16_t*>(d_k);
  a.av = static_cast<const uint16_t*>(d_v);
  a.wtail_k = const_cast<uint16_t*>(a.tail_k);
  a.wtail_v = const_cast<uint16_t*>(a.tail_v);
  a.an_max = n_max;
  hipError_t e = fmt == qs::kFmtNibble
                     ? qs::launch_attention_app(a, cf.head_dim, draft, static_cast<hipStream_t>(stream))
                     : qs::launch_attention_app_split(a, cf.head_dim, draft,
                                                      static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_fail(c, e, draft ? "draft launch" : "verify launch");
  c->st.apply_append(layer, n);
  c->err.clear();
  return QS_OK;
}

qs_status qs_attend_draft(qs_cache* c, int32_t layer, const void* d_q, float sm_scale, float* d_out,
                          void* stream) {
  return attend(c, layer, d_q, 1, sm_scale, d_out, stream, true);
}

qs_status qs_attend_verify(qs_cache* c, int32_t layer, const void* d_q, int32_t m, float sm_scale,
                           float* d_out, void* stream) {
  return attend(c, layer, d_q, m, sm_scale, d_out, stream, false);
}

qs_status qs_attend_draft_bits(qs_cache* c, int32_t layer, const void* d_q, int32_t bits,
                               float sm_scale, float* d_out, void* stream) {
  return attend(c, layer, d_q, 1, sm_scale, d_out, stream, true, bits);
}

qs_status qs_attend_draft_gqa(qs_cache* c, int32_t layer, const void* d_q, int32_t g,
                              float sm_scale, float* d_out, void* stream) {
  return attend_gqa(c, layer, d_q, 1, g, sm_scale, d_out, stream, true);
}

qs_status qs_attend_verify_gqa(qs_cache* c, int32_t layer, const void* d_q, int32_t m, int32_t g,
                               float sm_scale, float* d_out, void* stream) {
  return attend_gqa(c, layer, d_q, m, g, sm_scale, d_out, stream, false);
}

qs_status qs_append_attend_draft(qs_cache* c, int32_t layer, const void* d_k, const void* d_v,
                                 int32_t n_max, const int32_t* h_n, const void* d_q,
                                 float sm_scale, float* d_out, void* stream) {
  return append_attend(c, layer, d_k, d_v, n_max, h_n, d_q, 1, sm_scale, d_out, stream, true);
}

qs_status qs_append_attend_verify(qs_cache* c, int32_t layer, const void* d_k, const void* d_v,
                                  const void* d_q, int32_t m, float sm_scale, float* d_out,
                                  void* stream) {
  if (c && (m < 1 || m > c->cfg.gamma_max + 1))
    return fail(c, QS_ERR_INVALID_ARG, "m must be in 1..gamma_max+1");
  return append_attend(c, layer, d_k, d_v, m, nullptr, d_q, m, sm_scale, d_out, stream, false);
}

qs_status qs_get_state(const qs_cache* c, int32_t layer, int32_t* h_nq, int32_t* h_nt, int32_t* h_head) {
  if (!c || layer < 0 || layer >= c->cfg.n_layers) return QS_ERR_INVALID_ARG;
  if (c->dev) return QS_ERR_STATE;
  for (int b = 0; b < c->cfg.batch; ++b) {
    const qs::Seq& s = c->st.at(layer, b);
    if (h_nq) h_nq[b] = s.nq;
    if (h_nt) h_nt[b] = s.nt;
    if (h_head) h_head[b] = s.head;
  }
  return QS_OK;
}

// ---- device mode ---------------------------------------------------------------------------

qs_status qs_state_to_device(qs_cache* c, void* stream) {
  if (!c) return QS_ERR_INVALID_ARG;
  if (c->dev) return fail(c, QS_ERR_STATE, "already in device mode");
  if (c->cfg.split_upper) return fail(c, QS_ERR_INVALID_ARG, kNotSplit);
  const qs_config& cf = c->cfg;
  const size_t n = (size_t)cf.n_layers * cf.batch;
  std::vector<int32_t> h(n * qs::kStateInts + 1, 0);
  for (int l = 0; l < cf.n_layers; ++l)
    for (int b = 0; b < cf.batch; ++b) {
      const qs::Seq& q = c->st.at(l, b);
      int32_t* e = &h[((size_t)l * cf.batch + b) * qs::kStateInts];
      e[0] = q.nq;
      e[1] = q.nt;
      e[2] = q.head;
    }
  const hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(dev_state(c), h.data(), h.size() * sizeof(int32_t),
                                hipMemcpyHostToDevice, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return device_fail(c, e, "state to device");
  c->dev = true;
  c->pend.assign(cf.n_layers, qs::Pending{});
  c->err.clear();
  return QS_OK;
}

static qs::StateArgs state_args(const qs_cache* c, int op, int l0, int nl) {
  qs::StateArgs a{};
  a.state = dev_state(c);
  a.err = dev_error(c);
  a.op = op;
  a.l0 = l0;
  a.nl = nl;
  a.B = c->cfg.batch;
  a.G = c->cfg.group;
  a.T = c->cfg.max_ctx;
  return a;
}

// Writes the pending operations of layers l0 .. l1-1 to the state section (one small launch per
// layer that has any).
static hipError_t commit_layers(qs_cache* c, int l0, int l1, hipStream_t st) {
  for (int l = l0; l < l1; ++l) {
    if (c->pend[l].count == 0) continue;
    qs::StateArgs sa = state_args(c, 0, l, 1);
    sa.pend = c->pend[l];
    hipError_t e = qs::launch_state(sa, st);
    if (e != hipSuccess) return e;
    c->pend[l] = qs::Pending{};
  }
  return hipSuccess;
}

static bool same_pending(const qs::Pending& x, const qs::Pending& y) {
  if (x.count != y.count) return false;
  for (int k = 0; k < x.count; ++k)
    if (x.op[k].kind != y.op[k].kind || x.op[k].n != y.op[k].n || x.op[k].sub != y.op[k].sub)
      return false;
  return true;
}

// Records an operation of `layer`, committing the full list first if needed.
static hipError_t push_pending(qs_cache* c, int layer, qs::PendingOp op, hipStream_t st) {
  if (c->pend[layer].count == qs::kMaxPending) {
    hipError_t e = commit_layers(c, layer, layer + 1, st);
    if (e != hipSuccess) return e;
  }
  qs::Pending& p = c->pend[layer];
  p.op[p.count++] = op;
  return hipSuccess;
}

qs_status qs_commit_dev(qs_cache* c, int32_t layer, void* stream) {
  if (!c) return QS_ERR_INVALID_ARG;
  if (!c->dev) return fail(c, QS_ERR_STATE, kInHostMode);
  if (layer < -1 || layer >= c->cfg.n_layers) return fail(c, QS_ERR_INVALID_ARG, "layer out of range");
  const int l0 = layer < 0 ? 0 : layer, l1 = layer < 0 ? c->cfg.n_layers : layer + 1;
  hipError_t e = commit_layers(c, l0, l1, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_fail(c, e, "state launch");
  c->err.clear();
  return QS_OK;
}

qs_status qs_state_from_device(qs_cache* c, void* stream, int32_t* h_error) {
  if (!c) return QS_ERR_INVALID_ARG;
  if (!c->dev) return fail(c, QS_ERR_STATE, kInHostMode);
  const qs_config& cf = c->cfg;
  {
    hipError_t e = commit_layers(c, 0, cf.n_layers, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return device_fail(c, e, "state launch");
  }
  const size_t n = (size_t)cf.n_layers * cf.batch;
  std::vector<int32_t> h(n * qs::kStateInts + 1, 0);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(h.data(), dev_state(c), h.size() * sizeof(int32_t),
                                hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return device_fail(c, e, "state from device");
  for (size_t i = 0; i < n; ++i) {  // the device keeps these invariants; check before adopting
    const int32_t* q = &h[i * qs::kStateInts];
    if (q[0] < 0 || q[0] > cf.max_ctx || q[0] % cf.group || q[1] < 0 || q[1] > 2 * cf.group ||
        (q[2] != 0 && q[2] != cf.group))
      return fail(c, QS_ERR_DEVICE, "device counters out of range");
  }
  for (int l = 0; l < cf.n_layers; ++l)
    for (int b = 0; b < cf.batch; ++b) {
      const int32_t* q = &h[((size_t)l * cf.batch + b) * qs::kStateInts];
      qs::Seq& s = c->st.at(l, b);
      s.nq = q[0];
      s.nt = q[1];
      s.head = q[2];
    }
  if (h_error) *h_error = h[n * qs::kStateInts];
  c->dev = false;
  c->err.clear();
  return QS_OK;
}

qs_status qs_append_dev(qs_cache* c, int32_t layer, const void* d_k, const void* d_v, int32_t n,
                        void* stream) {
  if (!c) return QS_ERR_INVALID_ARG;
  if (!c->dev) return fail(c, QS_ERR_STATE, kInHostMode);
  const qs_config& cf = c->cfg;
  if (layer < 0 || layer >= cf.n_layers) return fail(c, QS_ERR_INVALID_ARG, "layer out of range");
  if (n < 0 || n > 2 * cf.group) return fail(c, QS_ERR_INVALID_ARG, "n must be in 0..2G");
  if (!d_k || !d_v) return fail(c, QS_ERR_INVALID_ARG, "null k or v");
  if (n == 0) return QS_OK;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  qs::AppendArgs a{};
  a.k = static_cast<const uint16_t*>(d_k);
  a.v = static_cast<const uint16_t*>(d_v);
  const size_t tail_lbh = (size_t)2 * cf.group * cf.head_dim * 2;
  a.tail_k = reinterpret_cast<uint16_t*>(c->arena + c->lay.tail_k + layer_off(c, tail_lbh, layer));
  a.tail_v = reinterpret_cast<uint16_t*>(c->arena + c->lay.tail_v + layer_off(c, tail_lbh, layer));
  a.B = cf.batch;
  a.H = cf.n_heads;
  a.n_max = n;
  a.n_rows = n;
  a.dstate = dev_state(c) + (size_t)layer * cf.batch * qs::kStateInts;
  for (int b = 0; b < cf.batch; ++b) a.n[b] = n;
  if (c->pend[layer].count == qs::kMaxPending) {  // room for this append's own entry
    hipError_t e = commit_layers(c, layer, layer + 1, st);
    if (e != hipSuccess) return device_fail(c, e, "state launch");
  }
  a.pend = c->pend[layer];
  hipError_t e = qs::launch_append(a, cf.head_dim, st);
  if (e != hipSuccess) return device_fail(c, e, "append launch");
  e = push_pending(c, layer, qs::PendingOp{0, n, nullptr}, st);
  if (e != hipSuccess) return device_fail(c, e, "state launch");
  c->err.clear();
  return QS_OK;
}

qs_status qs_rollback_dev(qs_cache* c, int32_t layer, int32_t n, const int32_t* d_sub,
                          void* stream) {
  if (!c) return QS_ERR_INVALID_ARG;
  if (!c->dev) return fail(c, QS_ERR_STATE, kInHostMode);
  const qs_config& cf = c->cfg;
  if (layer < -1 || layer >= cf.n_layers) return fail(c, QS_ERR_INVALID_ARG, "layer out of range");
  if (n < 0) return fail(c, QS_ERR_INVALID_ARG, "n must be >= 0");
  const int l0 = layer < 0 ? 0 : layer, l1 = layer < 0 ? cf.n_layers : layer + 1;
  for (int l = l0; l < l1; ++l) {
    hipError_t e = push_pending(c, l, qs::PendingOp{1, n, d_sub}, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return device_fail(c, e, "state launch");
  }
  c->err.clear();
  return QS_OK;
}

qs_status qs_flush_dev(qs_cache* c, int32_t layer, int32_t min_tail, void* stream) {
  if (!c) return QS_ERR_INVALID_ARG;
  if (!c->dev) return fail(c, QS_ERR_STATE, kInHostMode);
  const qs_config& cf = c->cfg;
  if (layer < -1 || layer >= cf.n_layers) return fail(c, QS_ERR_INVALID_ARG, "layer out of range");
  if (min_tail > 2 * cf.group) return fail(c, QS_ERR_INVALID_ARG, "min_tail must be <= 2G");
  const int l0 = layer < 0 ? 0 : layer, nl = layer < 0 ? cf.n_layers : 1;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  // one launch serves layers with the same pending operations; otherwise commit them first
  for (int l = l0 + 1; l < l0 + nl; ++l)
    if (!same_pending(c->pend[l], c->pend[l0])) {
      hipError_t e = commit_layers(c, l0, l0 + nl, st);
      if (e != hipSuccess) return device_fail(c, e, "state launch");
      break;
    }
  qs::FlushArgs a{};
  a.uk = c->arena + c->lay.uk;
  a.lk = c->arena + c->lay.lk;
  a.uv = c->arena + c->lay.uv;
  a.lv = c->arena + c->lay.lv;
  a.kmeta = c->arena + c->lay.kmeta;
  a.vmeta = c->arena + c->lay.vmeta;
  a.meta16 = cf.meta_fp16;
  a.split = cf.split_upper;
  a.tail_k = reinterpret_cast<const uint16_t*>(c->arena + c->lay.tail_k);
  a.tail_v = reinterpret_cast<const uint16_t*>(c->arena + c->lay.tail_v);
  a.B = cf.batch;
  a.H = cf.n_heads;
  a.T = cf.max_ctx;
  a.NG = cf.max_ctx / cf.group;
  a.layer0 = l0;
  a.n_sel = cf.batch;
  for (int b = 0; b < cf.batch; ++b) a.b[b] = b;
  a.dstate = dev_state(c);
  a.thr = c->st.flush_threshold(min_tail);
  a.pend = c->pend[l0];
  hipError_t e = qs::launch_flush(a, cf.head_dim, nl, st);
  if (e != hipSuccess) return device_fail(c, e, "flush launch");
  qs::StateArgs sa = state_args(c, 1, l0, nl);
  sa.thr = a.thr;
  sa.pend = c->pend[l0];
  e = qs::launch_state(sa, st);
  if (e != hipSuccess) return device_fail(c, e, "state launch");
  for (int l = l0; l < l0 + nl; ++l) c->pend[l] = qs::Pending{};
  c->err.clear();
  return QS_OK;
}

static qs_status attend_dev(qs_cache* c, int32_t layer, const void* d_q, int32_t m, float sm_scale,
                            float* d_out, void* stream, bool draft) {
  if (!c) return QS_ERR_INVALID_ARG;
  if (!c->dev) return fail(c, QS_ERR_STATE, kInHostMode);
  const qs_config& cf = c->cfg;
  if (layer < 0 || layer >= cf.n_layers) return fail(c, QS_ERR_INVALID_ARG, "layer out of range");
  if (!draft && (m < 1 || m > cf.gamma_max + 1))
    return fail(c, QS_ERR_INVALID_ARG, "m must be in 1..gamma_max+1");
  if (!d_q || !d_out) return fail(c, QS_ERR_INVALID_ARG, "null q or out");
  if (!isfinite(sm_scale)) return fail(c, QS_ERR_INVALID_ARG, "sm_scale must be finite");
  // a plan that holds for any counters: kMaxTailItems tail items per sequence and head, and W
  // quantized workers filling the rest of one resident round (worker w takes groups w, w + W,
  // .. of whatever the sequence holds).  Tail items past nt exit at once, so they are counted
  // as half their number.  Workers and items with no work write empty records.
  int slots = qs::attention_slots(cf.head_dim, draft, cf.batch, qs::kModeDev, cf.meta_fp16 != 0,
                                  qs::kFmtNibble);
  if (slots <= 0) slots = kFallbackSlots;
  const int bh = cf.batch * cf.n_heads;
  int W = (slots - bh * qs::kMaxTailItems / 2) / bh;
  W = W < 1 ? 1 : (W > qs::kMaxQuantSplits ? qs::kMaxQuantSplits : W);
  const int NG = cf.max_ctx / cf.group;
  if (W > NG) W = NG;
  qs::Plan p;
  p.chunk_groups = (NG + W - 1) / W;
  for (int b = 0; b < cf.batch; ++b) {
    p.qitems[b] = W;
    p.titems[b] = qs::kMaxTailItems;
    p.qbase[b + 1] = p.qbase[b] + W;
    p.tbase[b + 1] = p.tbase[b] + qs::kMaxTailItems;
  }
  qs::AttnDevArgs a{};
  attn_args(c, layer, d_q, m, sm_scale, d_out, p, a);
  a.dev.dstate = dev_state(c) + (size_t)layer * cf.batch * qs::kStateInts;
  a.dev.wstate = dev_state(c) + (size_t)layer * cf.batch * qs::kStateInts;
  a.dev.derr = dev_error(c);
  a.dev.min_nt = draft ? 0 : m;
  a.dev.pend = c->pend[layer];
  hipError_t e = qs::launch_attention_dev(a, cf.head_dim, draft, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_fail(c, e, draft ? "draft launch" : "verify launch");
  c->pend[layer] = qs::Pending{};  // committed by the combine kernel
  c->err.clear();
  return QS_OK;
}

qs_status qs_attend_draft_dev(qs_cache* c, int32_t layer, const void* d_q, float sm_scale,
                              float* d_out, void* stream) {
  return attend_dev(c, layer, d_q, 1, sm_scale, d_out, stream, true);
}

qs_status qs_attend_verify_dev(qs_cache* c, int32_t layer, const void* d_q, int32_t m,
                               float sm_scale, float* d_out, void* stream) {
  return attend_dev(c, layer, d_q, m, sm_scale, d_out, stream, false);
}

const char* qs_last_error(const qs_cache* c) { return c ? c->err.c_str() : "null cache"; }

}  // extern "C"
