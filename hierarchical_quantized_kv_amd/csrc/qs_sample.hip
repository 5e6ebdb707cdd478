// qs_sample.hip -- the speculative accept / correct step after the verify pass (gfx950).
//
// Per sequence b, with target logits t_i (rows i = 0 .. gamma, the target's next-token scores at
// the gamma drafted positions and one past them), draft logits d_i (rows i = 0 .. gamma-1) and
// the gamma drafted tokens x_i:
//   p_i = softmax(t_i),  q_i = softmax(d_i)
//   drafted token i is accepted iff u_i <= min(1, p_i(x_i) / (q_i(x_i) + 1e-8)), scanning
//   i = 0, 1, .. and stopping at the first rejection j;
//   the next token is sampled with u_gamma from (p_j - q_j)_+ normalised if a token was rejected
//   at j, else from p_gamma.
// [QuantSpec Guide, "The Self-Speculative Verification Loop" listing: the acceptance test;
// Pith review of arXiv:2502.10424, major comment 1 on Algorithm 1: VERIFY accepts with
// min(1, p/q) and CORRECT samples from the normalised residual (p - q)_+; minor comment 5: after
// gamma acceptances the next token comes from p_{gamma+1}.]
//
// Three launches, all fp32:
//   row_stats_kernel  (max, sum of exp(x - max)) of every row in parts of 4096 tokens, one
//                     workgroup per (row, part);
//   part_sums_kernel  per part of a sequence: every row's statistics merged, the acceptance
//                     tests (so the rejection point j), then the part's totals of the sampling
//                     weights for that j only ((p_j - q_j)_+, or p_gamma, and p_j itself); part
//                     0 also stores the row statistics and the acceptance ratios;
//   accept_kernel     per sequence: the acceptance tests (one lane per drafted token, the first
//                     failure is j), then the inverse CDF: the part from a scan of the part totals of the chosen j, the
//                     token from one recomputation of that part.
// So the whole vocabulary is read once by many workgroups in parallel, then the one or two rows
// of the rejection point once more, and the one workgroup per sequence reads only 4096 tokens
// of two rows.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "../../include/quantspec.h"

namespace qs_sample {

constexpr int kPartThreads = 256;                 // one workgroup per row part of kPartTokens
constexpr int kPartPer = 16;                      //   consecutive tokens, kPartPer per thread
constexpr int kPartTokens = kPartThreads * kPartPer;
constexpr int kWaves = kPartThreads / 64;
constexpr int kMaxParts = 256;                    // vocab <= kMaxParts * kPartTokens = 1048576

__host__ __device__ inline int row_parts(int V) { return (V + kPartTokens - 1) / kPartTokens; }

// Workspace, in floats, for B sequences, gamma drafted tokens and np = row_parts(V):
//   part_stat [B][2 gamma + 1][np][2]  (max, sum of exp(x - max)) per row part; rows 0 .. gamma
//                                      are the target rows, gamma+1 .. 2 gamma the draft rows
//   row_stat  [B][2 gamma + 1][2]      (max, 1 / sum) per row
//   part_sum  [B][np][2]               for the sequence's rejection point j: the part's total of
//                                      the sampling weight ((p_j - q_j)_+ for j < gamma, p_gamma
//                                      for j = gamma) and of p_j
//   ratio     [B][gamma]               min(1, p_i(x_i) / (q_i(x_i) + 1e-8)), or -1 for a drafted
//                                      token outside the vocabulary
//   xlogit    [B][gamma][2]            the target and draft logits of drafted token x_i (rows i
//                                      and gamma+1+i), stored by the row-statistics pass (not
//                                      written for a token outside the vocabulary)
struct WsLayout {
  size_t part_stat, row_stat, part_sum, ratio, xlogit, total;
};
__host__ __device__ inline WsLayout ws_layout(int B, int gamma, int np) {
  WsLayout L;
  const size_t rows = (size_t)B * (2 * gamma + 1);
  L.part_stat = 0;
  L.row_stat = L.part_stat + rows * np * 2;
  L.part_sum = L.row_stat + rows * 2;
  L.ratio = L.part_sum + (size_t)B * np * 2;
  L.xlogit = L.ratio + (size_t)B * gamma;
  L.total = L.xlogit + (size_t)B * gamma * 2;
  return L;
}

struct RowStat {
  float m, s;  // max and sum of exp(x - max) of a row (part)
};

__device__ __forceinline__ RowStat merge(RowStat a, RowStat b) {
  const float m = fmaxf(a.m, b.m);
  if (m == -INFINITY) return RowStat{-INFINITY, 0.f};
  return RowStat{m, a.s * expf(a.m - m) + b.s * expf(b.m - m)};
}

// The kPartPer logits of this thread in part `part` of a row (-inf past V), in one of two orders
// (the row statistics and the part totals do not depend on it): with vec, 16-byte loads, thread
// t holding tokens 4 (t + 256 k) + e; else tokens t + 256 k.  vec needs a 16-byte aligned row
// and V a multiple of 4 (then 4 (t + 256 k) < V implies the three tokens after it are too).
__device__ __forceinline__ bool vec_ok(const float* row, int V) {
  return (V & 3) == 0 && ((uintptr_t)row & 15) == 0;
}
__device__ __forceinline__ void load_part_any(const float* row, int V, int part, bool vec,
                                              float (&x)[kPartPer]) {
  const int base = part * kPartTokens;
  if (vec) {
    const float4* r4 = reinterpret_cast<const float4*>(row + base);
    float4 q[kPartPer / 4];
#pragma unroll
    for (int k = 0; k < kPartPer / 4; ++k) {
      const int i = k * kPartThreads + (int)threadIdx.x;
      q[k] = base + 4 * i < V ? r4[i] : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
    }
#pragma unroll
    for (int k = 0; k < kPartPer / 4; ++k) {
      x[4 * k] = q[k].x;
      x[4 * k + 1] = q[k].y;
      x[4 * k + 2] = q[k].z;
      x[4 * k + 3] = q[k].w;
    }
  } else {
#pragma unroll
    for (int k = 0; k < kPartPer; ++k) {
      const int v = base + k * kPartThreads + (int)threadIdx.x;
      x[k] = v < V ? row[v] : -INFINITY;
    }
  }
}

// grid: x = row (0 .. gamma: target rows, gamma+1 .. 2 gamma: draft rows), y = part, z = sequence.
// Coalesced, all loads first.  The sums use the hardware exp2 (a few ulp per term).  The thread
// that holds the logit of the row's drafted token (rows i < gamma and gamma+1+i: token x_i)
// also stores it for the acceptance test.
__global__ __launch_bounds__(kPartThreads) void row_stats_kernel(const float* __restrict__ t,
                                                                 const float* __restrict__ d,
                                                                 const int32_t* __restrict__ tokens,
                                                                 int gamma, int V, float* ws) {
  __shared__ RowStat sh[kPartThreads / 64];
  const int r = blockIdx.x, part = blockIdx.y, b = blockIdx.z;
  const float* row = r <= gamma ? t + ((size_t)b * (gamma + 1) + r) * V
                                : d + ((size_t)b * gamma + (r - gamma - 1)) * V;
  const int di = r < gamma ? r : r - gamma - 1;  // the drafted token of this row, or -1
  const int xtok = di >= 0 ? tokens[(size_t)b * gamma + di] : -1;
  const bool vec = vec_ok(row, V);
  float x[kPartPer];
  load_part_any(row, V, part, vec, x);
  {
    const int off = xtok - part * kPartTokens;
    if (xtok >= 0 && xtok < V && off >= 0 && off < kPartTokens) {
      // the token's thread and slot in load_part_any's order
      const int owner = vec ? ((off >> 2) & (kPartThreads - 1)) : (off & (kPartThreads - 1));
      const int slot = vec ? ((off >> 10) * 4 + (off & 3)) : (off >> 8);
      if ((int)threadIdx.x == owner) {
        float val = x[0];
#pragma unroll
        for (int k = 1; k < kPartPer; ++k)
          if (k == slot) val = x[k];
        const WsLayout L = ws_layout(gridDim.z, gamma, row_parts(V));
        ws[L.xlogit + ((size_t)b * gamma + di) * 2 + (r < gamma ? 0 : 1)] = val;
      }
    }
  }
  float m = x[0];
#pragma unroll
  for (int k = 1; k < kPartPer; ++k) m = fmaxf(m, x[k]);
  float sum = 0.f;
  if (m != -INFINITY) {
#pragma unroll
    for (int k = 0; k < kPartPer; ++k)
      sum += __builtin_amdgcn_exp2f((x[k] - m) * 1.4426950408889634f);
  }
  RowStat st{m, sum};
  for (int o = 32; o > 0; o >>= 1)
    st = merge(st, RowStat{__shfl_xor(st.m, o), __shfl_xor(st.s, o)});
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = st;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kPartThreads / 64; ++w) st = merge(st, sh[w]);
    float* o = ws + (((size_t)b * (2 * gamma + 1) + r) * row_parts(V) + part) * 2;
    o[0] = st.m;
    o[1] = st.s;
  }
}

__device__ __forceinline__ float prob(float x, float2 st) {
  return st.y > 0.f ? expf(x - st.x) * st.y : 0.f;
}

// Sampling weights use the hardware exp2 (a few ulp): the sample is an inverse CDF over up to a
// million weights summed in fp32, far coarser than that.
__device__ __forceinline__ float prob_fast(float x, float2 st) {
  return st.y > 0.f ? __builtin_amdgcn_exp2f((x - st.x) * 1.4426950408889634f) * st.y : 0.f;
}

// Exclusive prefix of x >= 0 over the workgroup's kPartThreads threads in thread order, into
// ex[tid]; ex[kPartThreads] receives the total.  ex is non-decreasing (each entry is the rounded
// inclusive prefix of the previous thread), so [ex[t], ex[t+1]) tile [0, total) without gaps;
// the same inputs give the same outputs on every call.
__device__ void block_exclusive_scan(float x, float* ex, float* wsum) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  float inc = x;
  for (int o = 1; o < 64; o <<= 1) {
    const float y = __shfl_up(inc, o);
    if (lane >= o) inc += y;
  }
  float exc = __shfl_up(inc, 1);
  if (lane == 0) exc = 0.f;
  if (lane == 63) wsum[w] = inc;
  __syncthreads();
  if (tid == 0) {
    float run = 0.f;
    for (int k = 0; k < kWaves; ++k) {
      const float v = wsum[k];
      wsum[k] = run;
      run += v;
    }
    ex[kPartThreads] = run;
  }
  __syncthreads();
  ex[tid] = wsum[w] + exc;
  __syncthreads();
}

// Cross-lane steps with DPP inside rows of 16 lanes: quad_perm swaps inside groups of four, the
// mirrors inside half rows and rows (for a max or a sum over a row, a mirror serves as well as
// an exchange).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

// Row statistics (max, 1 / sum) of the R = 2 gamma + 1 rows of sequence b, merged from their
// parts into out[r]: wave w takes rows w, w + kWaves, .. (all of its loads issued first), lane l
// the parts l, l + 64, .. (merged in order), then per row the largest max over the lanes
// holding parts, each lane's sum scaled to it once, and the scaled sums added.
constexpr int kMaxRows = 2 * (QS_MAX_QUERIES - 1) + 1;
constexpr int kRowsPerWave = (kMaxRows + kWaves - 1) / kWaves;
__device__ void merge_all_rows(const float* part_stat, int np, int R, float2* out) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  RowStat a[kRowsPerWave];
#pragma unroll
  for (int k = 0; k < kRowsPerWave; ++k) {
    const int r = wv + kWaves * k;
    a[k] = (r < R && lane < np) ? RowStat{part_stat[((size_t)r * np + lane) * 2],
                                          part_stat[((size_t)r * np + lane) * 2 + 1]}
                                : RowStat{-INFINITY, 0.f};
  }
  for (int p0 = 64; p0 < np; p0 += 64) {  // vocabularies above 64 parts
    const int pt = p0 + lane;
#pragma unroll
    for (int k = 0; k < kRowsPerWave; ++k) {
      const int r = wv + kWaves * k;
      if (r < R && pt < np)
        a[k] = merge(a[k], RowStat{part_stat[((size_t)r * np + pt) * 2],
                                   part_stat[((size_t)r * np + pt) * 2 + 1]});
    }
  }
  // lanes at or past np hold (-inf, 0), so lane 0 needs only the lanes below np: DPP steps
  // within the first 16 lanes, then shuffles across rows of 16 lanes when there are more parts;
  // every row of the wave goes through each step before the next
  float m[kRowsPerWave], sum[kRowsPerWave];
#pragma unroll
  for (int k = 0; k < kRowsPerWave; ++k) m[k] = a[k].m;
#pragma unroll
  for (int k = 0; k < kRowsPerWave; ++k) m[k] = fmaxf(m[k], dpp<kDppXor1>(m[k]));
#pragma unroll
  for (int k = 0; k < kRowsPerWave; ++k) m[k] = fmaxf(m[k], dpp<kDppXor2>(m[k]));
#pragma unroll
  for (int k = 0; k < kRowsPerWave; ++k) m[k] = fmaxf(m[k], dpp<kDppHalfMirror>(m[k]));
#pragma unroll
  for (int k = 0; k < kRowsPerWave; ++k) m[k] = fmaxf(m[k], dpp<kDppMirror>(m[k]));
  if (np > 16) {
#pragma unroll
    for (int k = 0; k < kRowsPerWave; ++k) m[k] = fmaxf(m[k], __shfl_xor(m[k], 16));
#pragma unroll
    for (int k = 0; k < kRowsPerWave; ++k) m[k] = fmaxf(m[k], __shfl_xor(m[k], 32));
  }
#pragma unroll
  for (int k = 0; k < kRowsPerWave; ++k)
    sum[k] = a[k].m == -INFINITY ? 0.f : a[k].s * expf(a[k].m - m[k]);
#pragma unroll
  for (int k = 0; k < kRowsPerWave; ++k) sum[k] += dpp<kDppXor1>(sum[k]);
#pragma unroll
  for (int k = 0; k < kRowsPerWave; ++k) sum[k] += dpp<kDppXor2>(sum[k]);
#pragma unroll
  for (int k = 0; k < kRowsPerWave; ++k) sum[k] += dpp<kDppHalfMirror>(sum[k]);
#pragma unroll
  for (int k = 0; k < kRowsPerWave; ++k) sum[k] += dpp<kDppMirror>(sum[k]);
  if (np > 16) {
#pragma unroll
    for (int k = 0; k < kRowsPerWave; ++k) sum[k] += __shfl_xor(sum[k], 16);
#pragma unroll
    for (int k = 0; k < kRowsPerWave; ++k) sum[k] += __shfl_xor(sum[k], 32);
  }
#pragma unroll
  for (int k = 0; k < kRowsPerWave; ++k) {
    const int r = wv + kWaves * k;
    if (lane == 0 && r < R) out[r] = make_float2(m[k], sum[k] > 0.f ? 1.f / sum[k] : 0.f);
  }
  __syncthreads();
}

// Weights of tokens part * kPartTokens + k * kPartThreads + tid (k < kPartPer): wp = p_j and
// wr = (p_j - q_j)_+, or wr = p_j when drow is null.  Tokens at or past V weigh 0.
__device__ __forceinline__ void part_weights(const float* trow, const float* drow, float2 pst,
                                             float2 qst, int V, int part, float (&wp)[kPartPer],
                                             float (&wr)[kPartPer]) {
  const int v0 = part * kPartTokens + (int)threadIdx.x;
  float xt[kPartPer], xd[kPartPer];
#pragma unroll
  for (int k = 0; k < kPartPer; ++k) {
    const int v = v0 + k * kPartThreads;
    xt[k] = v < V ? trow[v] : -INFINITY;
    xd[k] = (drow && v < V) ? drow[v] : -INFINITY;
  }
#pragma unroll
  for (int k = 0; k < kPartPer; ++k) {
    wp[k] = prob_fast(xt[k], pst);
    wr[k] = drow ? fmaxf(0.f, wp[k] - prob_fast(xd[k], qst)) : wp[k];
  }
}

// Totals of the kPartPer rows of a part (row k = the tokens of index k in every thread, in
// token order) into row_tot, and the part total (the rows in order).  Called by every thread.
// The rows pass through LDS: thread (k, c) sums columns c, c + 16, .. of row k, then thread k
// sums its row's 16 partial sums (the row stride is padded so that a wave's reads hit 64
// distinct banks).
constexpr int kRowPad = kPartThreads + 16;
__device__ float part_rows(const float (&w)[kPartPer], float* tile, float* partial,
                           float* row_tot) {
  static_assert(kPartPer * 16 == kPartThreads, "one thread per (row, column class)");
  const int tid = threadIdx.x;
#pragma unroll
  for (int k = 0; k < kPartPer; ++k) tile[k * kRowPad + tid] = w[k];
  __syncthreads();
  {
    const int k = tid >> 4, c = tid & 15;
    float x = 0.f;
#pragma unroll
    for (int i = 0; i < kPartThreads / 16; ++i) x += tile[k * kRowPad + c + 16 * i];
    partial[k * 17 + c] = x;
  }
  __syncthreads();
  if (tid < kPartPer) {
    float r = 0.f;
    for (int c = 0; c < 16; ++c) r += partial[tid * 17 + c];
    row_tot[tid] = r;
  }
  __syncthreads();
  float tot = 0.f;
  for (int k = 0; k < kPartPer; ++k) tot += row_tot[k];
  return tot;
}

// grid: x = part, y = sequence.  Every workgroup of a sequence merges the row statistics, takes
// the acceptance tests (the same fp32 operations on the same data in every workgroup, so all of
// them find the same j) and then sums the sampling weights of its part for that j only.
__global__ __launch_bounds__(kPartThreads) void part_sums_kernel(const float* __restrict__ t,
                                                                 const float* __restrict__ d,
                                                                 const int32_t* __restrict__ tokens,
                                                                 const float* __restrict__ u,
                                                                 int gamma, int V, float* ws) {
  __shared__ float2 rowst[kMaxRows];
  __shared__ float2 wsum[kWaves];
  __shared__ int s_j;
  const int part = blockIdx.x, b = blockIdx.y, B = gridDim.y;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int np = row_parts(V), R = 2 * gamma + 1;
  const WsLayout L = ws_layout(B, gamma, np);
  // the drafted tokens and their logits (lane i of wave 0: token i; the logits as the row
  // statistics pass stored them, read whatever the token so that no load waits on another)
  int x = -1;
  float tx = 0.f, dx = 0.f, ui = 0.f;
  if (tid < gamma) {
    x = tokens[(size_t)b * gamma + tid];
    tx = ws[L.xlogit + ((size_t)b * gamma + tid) * 2];
    dx = ws[L.xlogit + ((size_t)b * gamma + tid) * 2 + 1];
    ui = u[(size_t)b * (gamma + 1) + tid];
  }
  merge_all_rows(ws + L.part_stat + (size_t)b * R * np * 2, np, R, rowst);
  if (tid < 64) {
    // the acceptance ratio of drafted token i; a token outside the vocabulary is never
    // accepted (u >= 0 > -1)
    float acc = -1.f;
    if (tid < gamma && x >= 0 && x < V)
      acc = fminf(1.f, prob(tx, rowst[tid]) / (prob(dx, rowst[gamma + 1 + tid]) + 1e-8f));
    const bool ok = tid < gamma && ui <= acc;
    const unsigned long long fail = __ballot(tid < gamma && !ok);
    if (tid == 0) s_j = fail ? __ffsll((long long)fail) - 1 : gamma;
    if (part == 0 && tid < gamma) ws[L.ratio + (size_t)b * gamma + tid] = acc;
  }
  if (part == 0 && tid < R) {
    ws[L.row_stat + ((size_t)b * R + tid) * 2] = rowst[tid].x;
    ws[L.row_stat + ((size_t)b * R + tid) * 2 + 1] = rowst[tid].y;
  }
  __syncthreads();
  const int j = s_j;
  const float2 pst = rowst[j], qst = j < gamma ? rowst[gamma + 1 + j] : make_float2(0.f, 0.f);
  const float* trow = t + ((size_t)b * (gamma + 1) + j) * V;
  const float* drow = j < gamma ? d + ((size_t)b * gamma + j) * V : nullptr;
  // the part's totals, in any order (the sampler only uses them to pick a part and the point's
  // fraction of it): both rows in the same token order
  const bool vec = vec_ok(trow, V) && (!drow || vec_ok(drow, V));
  float xt[kPartPer], xd[kPartPer];
  load_part_any(trow, V, part, vec, xt);
  if (drow) load_part_any(drow, V, part, vec, xd);
  float sr = 0.f, sp = 0.f;
#pragma unroll
  for (int k = 0; k < kPartPer; ++k) {
    const float p = prob_fast(xt[k], pst);
    sp += p;
    sr += drow ? fmaxf(0.f, p - prob_fast(xd[k], qst)) : p;
  }
  for (int o = 32; o > 0; o >>= 1) {
    sr += __shfl_xor(sr, o);
    sp += __shfl_xor(sp, o);
  }
  if (lane == 0) wsum[wv] = make_float2(sr, sp);
  __syncthreads();
  if (tid == 0) {
    float2 tot = wsum[0];
    for (int w = 1; w < kWaves; ++w) {
      tot.x += wsum[w].x;
      tot.y += wsum[w].y;
    }
    float* o = ws + L.part_sum + ((size_t)b * np + part) * 2;
    o[0] = tot.x;
    o[1] = tot.y;
  }
}

// grid: x = sequence.
__global__ __launch_bounds__(kPartThreads) void accept_kernel(const float* __restrict__ t,
                                                              const float* __restrict__ d,
                                                              const float* __restrict__ u,
                                                              int gamma, int V,
                                                              const float* __restrict__ ws,
                                                              int32_t* n_accepted,
                                                              int32_t* next_token) {
  const int b = blockIdx.x, B = gridDim.x, tid = threadIdx.x;
  const int np = row_parts(V);
  const WsLayout L = ws_layout(B, gamma, np);
  const float* rs = ws + L.row_stat + (size_t)b * (2 * gamma + 1) * 2;
  const float* ub = u + (size_t)b * (gamma + 1);
  __shared__ float ex[kPartThreads + 1];
  __shared__ float wsum[kWaves];
  __shared__ float tile[kPartPer * kRowPad];
  __shared__ float partial[kPartPer * 17];
  __shared__ float row_tot[kPartPer];
  __shared__ int s_j, s_part, s_last_part, s_tok, s_row_last, s_part_last;
  // the part totals of the rejection point (j-independent slots), loaded with the tests' inputs
  const float* sums = ws + L.part_sum + (size_t)b * np * 2;
  const float sum_r = tid < np ? sums[2 * tid] : 0.f, sum_p = tid < np ? sums[2 * tid + 1] : 0.f;
  if (tid < 64) {  // wave 0: lane i tests drafted token i; j = the first one that fails
    const bool ok = tid < gamma && ub[tid] <= ws[L.ratio + (size_t)b * gamma + tid];
    const unsigned long long fail = __ballot(tid < gamma && !ok);
    if (tid == 0) {
      s_j = fail ? __ffsll((long long)fail) - 1 : gamma;
      s_part = -1;
      s_last_part = -1;
      s_tok = -1;
      s_row_last = -1;
      s_part_last = -1;
    }
  }
  __syncthreads();
  const int j = s_j;
  // the residual's part totals (p_gamma's when j = gamma); p_j's if the residual vanished in
  // rounding
  int plain = 0;
  float mine = sum_r;
  block_exclusive_scan(mine, ex, wsum);
  if (!(ex[kPartThreads] > 0.f)) {
    plain = 1;
    mine = sum_p;
    block_exclusive_scan(mine, ex, wsum);
  }
  const float total = ex[kPartThreads];
  if (!(total > 0.f)) {  // no positive weight at all (rows of -inf logits)
    if (tid == 0) {
      n_accepted[b] = j;
      next_token[b] = 0;
    }
    return;
  }
  // the part holding u * total, and the point's fraction of it; a point that rounding puts at
  // or past the total goes to the top of the last part of positive weight
  const float target = ub[gamma] * total;
  if (ex[tid] <= target && target < ex[tid + 1]) s_part = tid;
  if (mine > 0.f) atomicMax(&s_last_part, tid);
  __syncthreads();
  const int part = s_part >= 0 ? s_part : s_last_part;
  const float lo = ex[part], hi = ex[part + 1];
  const float frac = s_part >= 0 ? fminf(1.f, fmaxf(0.f, (target - lo) / (hi - lo))) : 1.f;
  // that part again: its rows, the row holding the point, then the token by a scan of the row
  const float* trow = t + ((size_t)b * (gamma + 1) + j) * V;
  const float* drow = (j < gamma && !plain) ? d + ((size_t)b * gamma + j) * V : nullptr;
  const int rq = 2 * (gamma + 1 + j);
  const float2 pst = make_float2(rs[2 * j], rs[2 * j + 1]);
  const float2 qst = j < gamma ? make_float2(rs[rq], rs[rq + 1]) : make_float2(0.f, 0.f);
  float wp[kPartPer], w[kPartPer];
  part_weights(trow, drow, pst, qst, V, part, wp, w);
  const float in_part = frac * part_rows(w, tile, partial, row_tot);
  float pre = 0.f;
  int row = 0;
  for (; row < kPartPer - 1; ++row) {
    if (row_tot[row] > 0.f && in_part - pre < row_tot[row]) break;
    pre += row_tot[row];
  }
  float wrow = 0.f;
  int last = -1;
#pragma unroll
  for (int k = 0; k < kPartPer; ++k) {
    if (k == row) wrow = w[k];
    if (w[k] > 0.f) last = part * kPartTokens + k * kPartThreads + tid;
  }
  if (last >= 0) atomicMax(&s_part_last, last);
  if (wrow > 0.f) atomicMax(&s_row_last, part * kPartTokens + row * kPartThreads + tid);
  block_exclusive_scan(wrow, ex, wsum);
  // the point within the row, in the scan's own units (its total and the row total differ by
  // rounding)
  const float rt = row_tot[row];
  const float rel = rt > 0.f ? fmaxf(0.f, fminf(in_part - pre, rt)) * (ex[kPartThreads] / rt) : 0.f;
  if (ex[tid] <= rel && rel < ex[tid + 1]) s_tok = part * kPartTokens + row * kPartThreads + tid;
  __syncthreads();
  if (tid == 0) {
    // a point at the very top of the row or part (rounding) takes the last token of positive
    // weight there
    n_accepted[b] = j;
    next_token[b] = s_tok >= 0 ? s_tok : s_row_last >= 0 ? s_row_last
                                      : s_part_last >= 0 ? s_part_last : 0;
  }
}

// Workspace of qs_spec_accept_static: a file-scope device array, one copy per GPU, held until
// the process ends.  Host code never uses its name as an address: the device address of each
// GPU's copy comes from hipGetSymbolAddress (scratch_ptr).
constexpr size_t kScratchBytes = size_t(4) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

// Device address of the current GPU's scratch array, looked up once per device (with that
// device current) and kept; null if the lookup fails.
void* scratch_ptr(hipError_t* err) {
  constexpr int kMaxDev = 64;
  static std::mutex mu;
  static void* ptr[kMaxDev] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDev) {
    *err = e != hipSuccess ? e : hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (!ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      *err = e != hipSuccess ? e : hipErrorInvalidSymbol;
      return nullptr;
    }
    ptr[dev] = p;
  }
  *err = hipSuccess;
  return ptr[dev];
}

}  // namespace qs_sample

extern "C" {

size_t qs_spec_workspace_bytes(int32_t batch, int32_t gamma, int32_t vocab) {
  if (batch < 1 || batch > 65535 || gamma < 1 || gamma + 1 > QS_MAX_QUERIES || vocab < 1 ||
      vocab > qs_sample::kMaxParts * qs_sample::kPartTokens)
    return 0;
  return qs_sample::ws_layout(batch, gamma, qs_sample::row_parts(vocab)).total * sizeof(float);
}

qs_status qs_spec_accept(const float* d_target_logits, const float* d_draft_logits,
                         const int32_t* d_draft_tokens, const float* d_uniforms, int32_t batch,
                         int32_t gamma, int32_t vocab, void* d_workspace, size_t workspace_bytes,
                         int32_t* d_n_accepted, int32_t* d_next_token, void* stream) {
  if (!d_target_logits || !d_draft_logits || !d_draft_tokens || !d_uniforms || !d_workspace ||
      !d_n_accepted || !d_next_token)
    return QS_ERR_INVALID_ARG;
  const size_t need = qs_spec_workspace_bytes(batch, gamma, vocab);
  if (need == 0) return QS_ERR_INVALID_ARG;
  if (workspace_bytes < need) return QS_ERR_BUFFER;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  float* ws = static_cast<float*>(d_workspace);
  const int np = qs_sample::row_parts(vocab);
  const dim3 block(qs_sample::kPartThreads);
  hipLaunchKernelGGL(qs_sample::row_stats_kernel, dim3(2 * gamma + 1, np, batch), block, 0, st,
                     d_target_logits, d_draft_logits, d_draft_tokens, gamma, vocab, ws);
  if (hipGetLastError() != hipSuccess) return QS_ERR_DEVICE;
  hipLaunchKernelGGL(qs_sample::part_sums_kernel, dim3(np, batch), block, 0, st, d_target_logits,
                     d_draft_logits, d_draft_tokens, d_uniforms, gamma, vocab, ws);
  if (hipGetLastError() != hipSuccess) return QS_ERR_DEVICE;
  hipLaunchKernelGGL(qs_sample::accept_kernel, dim3(batch), block, 0, st, d_target_logits,
                     d_draft_logits, d_uniforms, gamma, vocab, ws, d_n_accepted, d_next_token);
  if (hipGetLastError() != hipSuccess) return QS_ERR_DEVICE;
  return QS_OK;
}

qs_status qs_spec_accept_static(const float* d_target_logits, const float* d_draft_logits,
                                const int32_t* d_draft_tokens, const float* d_uniforms,
                                int32_t batch, int32_t gamma, int32_t vocab, int32_t* d_n_accepted,
                                int32_t* d_next_token, void* stream) {
  const size_t need = qs_spec_workspace_bytes(batch, gamma, vocab);
  if (need == 0) return QS_ERR_INVALID_ARG;
  if (need > qs_sample::kScratchBytes) return QS_ERR_BUFFER;
  hipError_t e = hipSuccess;
  void* ws = qs_sample::scratch_ptr(&e);
  if (!ws) return QS_ERR_DEVICE;
  return qs_spec_accept(d_target_logits, d_draft_logits, d_draft_tokens, d_uniforms, batch, gamma,
                        vocab, ws, qs_sample::kScratchBytes, d_n_accepted, d_next_token, stream);
}

}  // extern "C"
