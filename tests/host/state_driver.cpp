// Test driver of the library's host bookkeeping (qs_state.h), built with g++ on the CPU.
// Reads commands on stdin and prints, after each, the status and every layer's counters, so a
// Python test can replay the same script on the CPU oracle and compare.
//
//   create L B H D G T gamma off [meta_fp16]
//   append layer n_max n_0 .. n_{B-1}
//   prefill layer n_max n_0 .. n_{B-1}
//   rollback layer d_0 .. d_{B-1}
//   flush layer min_tail
//   attend layer m draft(0|1)
//   plan layer target_items          -> chunk_groups, then qitems[b] titems[b] pairs
//   layout                           -> section offsets and sizes
#include <cstdio>
#include <iostream>
#include <sstream>
#include <string>

#include "../../hierarchical_quantized_kv_amd/csrc/qs_state.h"

int main() {
  qs::State st;
  qs_config cfg{};
  std::string line;
  while (std::getline(std::cin, line)) {
    std::istringstream in(line);
    std::string op;
    in >> op;
    if (op.empty()) continue;
    std::string err;
    int status = 0;
    if (op == "create") {
      in >> cfg.n_layers >> cfg.batch >> cfg.n_heads >> cfg.head_dim >> cfg.group >> cfg.max_ctx >>
          cfg.gamma_max >> cfg.draft_offset;
      if (!(in >> cfg.meta_fp16)) cfg.meta_fp16 = 0;
      if (!qs::config_ok(cfg, &err)) {
        std::printf("status 1 %s\n", err.c_str());
        continue;
      }
      st = qs::State(cfg);
    } else if (op == "append") {
      int layer, n_max;
      in >> layer >> n_max;
      int32_t n[QS_MAX_BATCH];
      for (int b = 0; b < cfg.batch; ++b) in >> n[b];
      status = st.check_append(layer, n_max, n, &err);
      if (status == QS_OK) st.apply_append(layer, n);
    } else if (op == "prefill") {
      int layer, n_max;
      in >> layer >> n_max;
      int32_t n[QS_MAX_BATCH];
      for (int b = 0; b < cfg.batch; ++b) in >> n[b];
      status = st.check_prefill(layer, n_max, n, &err);
      if (status == QS_OK) st.apply_prefill(layer, n);
    } else if (op == "rollback") {
      int layer;
      in >> layer;
      int32_t d[QS_MAX_BATCH];
      for (int b = 0; b < cfg.batch; ++b) in >> d[b];
      status = st.check_rollback(layer, d, &err);
      if (status == QS_OK) st.apply_rollback(layer, d);
    } else if (op == "flush") {
      int layer, min_tail;
      in >> layer >> min_tail;
      status = st.check_flush(layer, min_tail, &err);
      if (status == QS_OK) {
        int l0 = layer < 0 ? 0 : layer, l1 = layer < 0 ? cfg.n_layers : layer + 1;
        for (int l = l0; l < l1; ++l)
          for (int b = 0; b < cfg.batch; ++b)
            if (st.selected(l, b, min_tail)) st.apply_flush_one(l, b);
      }
    } else if (op == "attend") {
      int layer, m, draft;
      in >> layer >> m >> draft;
      status = st.check_attend(layer, m, draft != 0, &err);
    } else if (op == "plan") {
      int layer, target;
      in >> layer >> target;
      qs::Seq s[QS_MAX_BATCH];
      for (int b = 0; b < cfg.batch; ++b) s[b] = st.at(layer, b);
      qs::Plan p = qs::make_plan(s, cfg.batch, cfg.n_heads, cfg.group, target);
      std::printf("plan %d", p.chunk_groups);
      for (int b = 0; b < cfg.batch; ++b) std::printf(" %d %d", p.qitems[b], p.titems[b]);
      std::printf("\n");
      continue;
    } else if (op == "layout") {
      qs_layout L = qs::make_layout(cfg);
      std::printf("layout %zu %zu %zu %zu %zu %zu %zu %zu %zu %zu %zu\n", L.uk, L.lk, L.uv, L.lv,
                  L.kmeta, L.vmeta, L.tail_k, L.tail_v, L.work, L.state, L.total);
      continue;
    } else {
      std::printf("status -1 unknown op\n");
      continue;
    }
    std::printf("status %d", status);
    for (int l = 0; l < cfg.n_layers; ++l)
      for (int b = 0; b < cfg.batch; ++b)
        std::printf(" %d,%d,%d", st.at(l, b).nq, st.at(l, b).nt, st.at(l, b).head);
    std::printf("\n");
  }
  return 0;
}
