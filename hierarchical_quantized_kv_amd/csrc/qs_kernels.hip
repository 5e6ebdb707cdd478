// qs_kernels.hip -- HIP kernels for gfx950 (MI355X) of the hierarchical INT8 KV cache.
//
// Kernels (one wave64 per work item unless noted):
//   append_kernel   fp16 rows -> tail ring slots
//   flush_kernel    oldest G-token ring half -> per-group asymmetric 8-bit codes, split into the
//                   upper / lower nibble planes, plus (scale, zero-point) metadata (256 threads)
//   attn_kernel     split-K attention work items of one pass:
//                     draft quantized item : upper key / value planes only, VALU (v_dot2)
//                     verify quantized item: both planes, MFMA 16x16x32 f16
//                     tail item            : up to 64 fp16 tail tokens, VALU, causal mask
//                   each writes one log-sum-exp partial (max, sum, o[D]) per query
//   combine_kernel  merges the partials of one (sequence, query, head)
//
// Sources: QuantSpec Guide (aifetchly), "Hierarchical Quantizer with Bit-Packing" listing
// (quantizer, unpack_for_draft, unpack_for_target); Pith review of arXiv:2502.10424, "What carries
// the argument" and Fig. 3 (C8 = 16*C_U + C_L, shared scale and zero-point), Fig. 7 and reference
// [128] (keys channel-wise, values token-wise; Flash-Decoding-compatible split softmax).
//
// Arithmetic of the quantized parts.  With per-channel key metadata (s_d, z_d) of the group and
// the query pre-scaled by sm_scale*log2(e):
//   draft score  = sum_d q_d s_d (16 U_d + off - z_d) = 16 sum_d q'_d U_d + sum_d q'_d (off - z_d)
//   verify score = sum_d q'_d C8_d - sum_d q'_d z_d,                 q'_d = q_d s_d
// and with per-token value metadata (s_t, z_t) and softmax weights p_t:
//   draft  o_d = 16 sum_t p'_t (U_td - 8) + sum_t p_t s_t (128 + off - z_t)
//   verify o_d =    sum_t p'_t (C8_td - 128) + sum_t p_t s_t (128 - z_t),   p'_t = p_t s_t
// The first sums run on fp16 operands built from the nibbles with the magic-number trick
// (0x6400 | n is the fp16 value 1024 + n); the second (bias) sums stay in fp32, which keeps
// degenerate groups (scale clamped to 1e-8, huge zero-point) exact.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "qs_args.h"

namespace qs {

typedef _Float16 f16;
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr uint32_t kMagic = 0x64006400u;  // two fp16 1024.0 with empty low mantissa bits

__device__ __forceinline__ f16x2 as_h2(uint32_t x) { return __builtin_bit_cast(f16x2, x); }
__device__ __forceinline__ uint32_t as_u32(f16x2 x) { return __builtin_bit_cast(uint32_t, x); }
__device__ __forceinline__ float dot2(f16x2 a, f16x2 b, float c) {
  return __builtin_amdgcn_fdot2(a, b, c, false);
}
__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ float lo_h(uint32_t x) { return (float)as_h2(x).x; }
__device__ __forceinline__ float hi_h(uint32_t x) { return (float)as_h2(x).y; }

// Word index and half of token/channel t inside a "pair-ordered" fp16 operand block: the
// nibbles of one 32-bit plane word w (8 entries, entry e in nibble e) come out as the fp16
// pairs (e0,e4) (e1,e5) (e2,e6) (e3,e7); the matching weights are stored in that order.
__device__ __forceinline__ int pair_word(int t) { return (t >> 3) * 4 + ((t & 7) & 3); }
__device__ __forceinline__ int pair_half(int t) { return (t & 7) >> 2; }

// 1024 + nibble pairs of one plane word, see pair_word().
struct Nib4 {
  f16x2 a, b, c, d;  // (e0,e4): 1024+n  (e1,e5): 1024+16n  (e2,e6): 1024+n  (e3,e7): 1024+16n
};
__device__ __forceinline__ Nib4 unpack_nibbles(uint32_t w) {
  Nib4 r;
  const uint32_t w8 = w >> 8;
  r.a = as_h2((w & 0x000F000Fu) | kMagic);
  r.b = as_h2((w & 0x00F000F0u) | kMagic);
  r.c = as_h2((w8 & 0x000F000Fu) | kMagic);
  r.d = as_h2((w8 & 0x00F000F0u) | kMagic);
  return r;
}

// 1024 + 16 * nibble for all 8 entries, pairs (e0,e4) (e1,e5) (e2,e6) (e3,e7): placing every
// nibble in mantissa bits 4-7 keeps the 1024 offset within a factor ~4 of the data.
__device__ __forceinline__ Nib4 unpack_nibbles16(uint32_t w) {
  Nib4 r;
  r.a = as_h2(((w << 4) & 0x00F000F0u) | kMagic);
  r.b = as_h2((w & 0x00F000F0u) | kMagic);
  r.c = as_h2(((w >> 4) & 0x00F000F0u) | kMagic);
  r.d = as_h2(((w >> 8) & 0x00F000F0u) | kMagic);
  return r;
}

// fp16 hi + lo split of x: hi = fp16(x), lo = fp16(x - hi); hi + lo carries ~22 bits.
__device__ __forceinline__ void split_f16(float x, f16& hi, f16& lo) {
  hi = (f16)x;
  lo = (f16)(x - (float)hi);
}

// 8-bit codes of 8 entries from an upper word u and lower word l (entry e in nibble e of each),
// as fp16 1024 + C8 in the slot order (e0,e2) (e4,e6) (e1,e3) (e5,e7).
__device__ __forceinline__ f16x8 codes_f16(uint32_t u, uint32_t l) {
  const uint32_t e = ((u << 4) & 0xF0F0F0F0u) | (l & 0x0F0F0F0Fu);  // C8 of e0 e2 e4 e6
  const uint32_t o = (u & 0xF0F0F0F0u) | ((l >> 4) & 0x0F0F0F0Fu);  // C8 of e1 e3 e5 e7
  uint32_t v0 = __builtin_amdgcn_perm(0x64646464u, e, 0x04010400u);
  uint32_t v1 = __builtin_amdgcn_perm(0x64646464u, e, 0x04030402u);
  uint32_t v2 = __builtin_amdgcn_perm(0x64646464u, o, 0x04010400u);
  uint32_t v3 = __builtin_amdgcn_perm(0x64646464u, o, 0x04030402u);
  f16x2 h0 = as_h2(v0), h1 = as_h2(v1), h2 = as_h2(v2), h3 = as_h2(v3);
  return f16x8{h0.x, h0.y, h1.x, h1.y, h2.x, h2.y, h3.x, h3.y};
}
// Slot s of codes_f16() holds entry kSigma[s].
// kSigma = {0, 2, 4, 6, 1, 3, 5, 7}

__device__ __forceinline__ float wave_max_from(float x, int from) {
  for (int o = from; o < 64; o <<= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum_from(float x, int from) {
  for (int o = from; o < 64; o <<= 1) x += __shfl_xor(x, o);
  return x;
}

// Record of split `split`, query `i` of (b, h).
__device__ __forceinline__ float* record(const AttnArgs& a, int D, int b, int h, int split, int i) {
  return a.work + ((((size_t)b * a.H + h) * a.S + split) * a.m + i) * (size_t)(D + kRecPad);
}

// ------------------------------------------------------------------------------------------
// Draft: quantized work item (upper planes only)
// ------------------------------------------------------------------------------------------

template <int D>
struct DraftShape {
  static constexpr int KL = D / 32;        // lanes per key row (16 bytes = 32 channels each)
  static constexpr int TPI = 64 / KL;      // key rows per load instruction
  static constexpr int KIT = kGroup / TPI; // key loads per lane per group
  static constexpr int VIT = D / 16;       // value loads per lane per group
};

struct DraftLds {
  uint32_t wts[2][64];   // key weights q' (hi, lo), pair order (D/2 words used)
  uint32_t pw[64];       // value weights p'_t, pair order (G/2 words)
  float2 vm[kGroup];     // (s_t, s_t * (128 + off - z_t))
};

template <int D>
__device__ void draft_quant_item(const AttnArgs& a, int b, int h, int item, DraftLds& L) {
  using S = DraftShape<D>;
  const int lane = threadIdx.x;
  const int ng = a.nq[b] / kGroup;
  const int g0 = item * a.chunk_groups;
  const int g1 = min(g0 + a.chunk_groups, ng);
  const size_t bh = (size_t)b * a.H + h;
  const float off = a.draft_offset;

  float q0 = 0.f, q1 = 0.f;  // channels 2*lane, 2*lane+1 (lanes < D/2), times qscale
  if (lane < D / 2) {
    const uint32_t qq = reinterpret_cast<const uint32_t*>(a.q + bh * D)[lane];
    q0 = lo_h(qq) * a.qscale;
    q1 = hi_h(qq) * a.qscale;
  }
  const int kc = lane % S::KL;   // key chunk (32 channels) of this lane
  const int kt = lane / S::KL;   // key row of this lane within a load
  const int vr = lane & 3;       // value quarter: tokens 32*vr .. 32*vr+31 of the group
  const int vd = lane >> 2;      // value channel offset: channel 16*i + vd

  float m_run = -INFINITY, l_run = 0.f, beta = 0.f;
  float acc[S::VIT];
#pragma unroll
  for (int i = 0; i < S::VIT; ++i) acc[i] = 0.f;

  for (int g = g0; g < g1; ++g) {
    const uint8_t* ukg = a.uk + (bh * a.T + (size_t)g * kGroup) * (D / 2);
    const uint8_t* uvg = a.uv + ((bh * a.NG + g) * D) * (kGroup / 2);
    uint4 kw[S::KIT], vw[S::VIT];
#pragma unroll
    for (int it = 0; it < S::KIT; ++it)
      kw[it] = ld16(ukg + (size_t)(it * S::TPI + kt) * (D / 2) + kc * 16);
#pragma unroll
    for (int i = 0; i < S::VIT; ++i)
      vw[i] = ld16(uvg + (size_t)(16 * i + vd) * (kGroup / 2) + vr * 16);
    float4 km = make_float4(0.f, 0.f, 0.f, 0.f);
    if (lane < D / 2)
      km = *reinterpret_cast<const float4*>(a.kmeta + (((bh * a.NG + g) * D) + 2 * lane) * 2);
    const float4 vm = *reinterpret_cast<const float4*>(a.vmeta + ((bh * a.T) + (size_t)g * kGroup + 2 * lane) * 2);

    __syncthreads();  // previous group's LDS reads are done
    // key weights q' = q s as fp16 hi + lo, against nibble values 1024 + 16 U
    float bias = 0.f;
    if (lane < D / 2) {
      const float qa = q0 * km.x, qb = q1 * km.z;
      f16 ah, al, bh, bl;
      split_f16(qa, ah, al);
      split_f16(qb, bh, bl);
      const int c0 = 2 * lane, c1 = 2 * lane + 1;
      f16* wh = reinterpret_cast<f16*>(L.wts[0]);
      f16* wl = reinterpret_cast<f16*>(L.wts[1]);
      wh[2 * pair_word(c0) + pair_half(c0)] = ah;
      wl[2 * pair_word(c0) + pair_half(c0)] = al;
      wh[2 * pair_word(c1) + pair_half(c1)] = bh;
      wl[2 * pair_word(c1) + pair_half(c1)] = bl;
      bias = qa * (off - km.y) + qb * (off - km.w) -
             1024.f * (((float)ah + (float)al) + ((float)bh + (float)bl));
    }
    L.vm[2 * lane] = make_float2(vm.x, vm.x * ((128.f + off) - vm.y));
    L.vm[2 * lane + 1] = make_float2(vm.z, vm.z * ((128.f + off) - vm.w));
    bias = wave_sum_from(bias, 1);
    __syncthreads();

    // scores of key rows it*TPI + kt
    uint4 W[4], Wl[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      W[k] = reinterpret_cast<const uint4*>(L.wts[0])[4 * kc + k];
      Wl[k] = reinterpret_cast<const uint4*>(L.wts[1])[4 * kc + k];
    }
    float sc[S::KIT];
#pragma unroll
    for (int it = 0; it < S::KIT; ++it) {
      const uint32_t wd[4] = {kw[it].x, kw[it].y, kw[it].z, kw[it].w};
      float p = 0.f;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const Nib4 n = unpack_nibbles16(wd[k]);
        p = dot2(n.a, as_h2(W[k].x), p);
        p = dot2(n.b, as_h2(W[k].y), p);
        p = dot2(n.c, as_h2(W[k].z), p);
        p = dot2(n.d, as_h2(W[k].w), p);
        p = dot2(n.a, as_h2(Wl[k].x), p);
        p = dot2(n.b, as_h2(Wl[k].y), p);
        p = dot2(n.c, as_h2(Wl[k].z), p);
        p = dot2(n.d, as_h2(Wl[k].w), p);
      }
#pragma unroll
      for (int o = 1; o < S::KL; o <<= 1) p += __shfl_xor(p, o);
      sc[it] = p + bias;
    }
    float gmax = sc[0];
#pragma unroll
    for (int it = 1; it < S::KIT; ++it) gmax = fmaxf(gmax, sc[it]);
    gmax = wave_max_from(gmax, S::KL);
    const float m_new = fmaxf(m_run, gmax);
    const float alpha = exp2f(m_run - m_new);
    m_run = m_new;
    l_run *= alpha;
    beta *= alpha;
#pragma unroll
    for (int i = 0; i < S::VIT; ++i) acc[i] *= alpha;
#pragma unroll
    for (int it = 0; it < S::KIT; ++it) {
      const int t = it * S::TPI + kt;
      const float p = exp2f(sc[it] - m_new);
      const float2 sw = L.vm[t];
      l_run += p;
      beta += p * sw.y;
      if (kc == 0)
        reinterpret_cast<f16*>(L.pw)[2 * pair_word(t) + pair_half(t)] =
            (f16)((t & 1) ? p * sw.x : 16.f * p * sw.x);
    }
    __syncthreads();

    // values: o_d += 16 p'_t (U_td - 8) over the 32 tokens of quarter vr
    uint4 P[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) P[k] = reinterpret_cast<const uint4*>(L.pw)[4 * vr + k];
    const f16x2 c1032 = {(f16)1032.f, (f16)1032.f}, c1152 = {(f16)1152.f, (f16)1152.f};
#pragma unroll
    for (int i = 0; i < S::VIT; ++i) {
      const uint32_t wd[4] = {vw[i].x, vw[i].y, vw[i].z, vw[i].w};
      float o = acc[i];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const Nib4 n = unpack_nibbles(wd[k]);
        o = dot2(n.a - c1032, as_h2(P[k].x), o);
        o = dot2(n.b - c1152, as_h2(P[k].y), o);
        o = dot2(n.c - c1032, as_h2(P[k].z), o);
        o = dot2(n.d - c1152, as_h2(P[k].w), o);
      }
      acc[i] = o;
    }
  }

  // l and beta were accumulated once per key row in each of its KL lanes
  l_run = wave_sum_from(l_run, S::KL);
  beta = wave_sum_from(beta, S::KL);
#pragma unroll
  for (int i = 0; i < S::VIT; ++i) {
    acc[i] += __shfl_xor(acc[i], 1);
    acc[i] += __shfl_xor(acc[i], 2);
  }
  float* rec = record(a, D, b, h, item, 0);
  if (lane == 0) {
    rec[0] = m_run;
    rec[1] = l_run;
  }
#pragma unroll
  for (int i = 0; i < S::VIT; ++i)
    if ((i & 3) == vr) rec[kRecPad + 16 * i + vd] = acc[i] + beta;
}

// ------------------------------------------------------------------------------------------
// Verify: quantized work item (both planes, MFMA)
// ------------------------------------------------------------------------------------------
//
// Per group of 128 tokens and lane l = 16*g + j (j: query column, g: k-group):
//   S^T tile tau (16 tokens x 16 queries) = sum over KK MFMAs of A (codes) x B (q' slots);
//   row r of tile tau is token 32*(r/4) + 8*(tau/2) + 2*(r%4) + (tau%2), so that lane group g
//   ends up holding exactly tokens 32g .. 32g+31 in the slot order PV needs.
//   O^T tile rt (16 channels x 16 queries) += A (value codes - 128) x B (p' of tiles 2q, 2q+1).

template <int D>
struct VerifyShape {
  static constexpr int KK = D / 32;   // MFMA k-steps per S^T tile
  static constexpr int CPL = D / 4;   // channels per lane group
  static constexpr int RT = D / 16;   // O^T channel tiles
};

struct VerifyLds {
  float2 km[128];        // (s_d, z_d) of the group's key channels
  float2 vm[kGroup];     // (s_t, s_t * (128 - z_t))
};

__device__ __forceinline__ int tile_row_token(int tau, int r) {
  return 32 * (r >> 2) + 8 * (tau >> 1) + 2 * (r & 3) + (tau & 1);
}

template <int D>
__device__ void verify_quant_item(const AttnArgs& a, int b, int h, int item, VerifyLds& L) {
  using S = VerifyShape<D>;
  const int lane = threadIdx.x;
  const int j = lane & 15;   // query
  const int g = lane >> 4;   // k-group
  const int m = a.m;
  const int ng = a.nq[b] / kGroup;
  const int g0 = item * a.chunk_groups;
  const int g1 = min(g0 + a.chunk_groups, ng);
  const size_t bh = (size_t)b * a.H + h;

  // this lane's query channels g*CPL .. g*CPL+CPL-1, times qscale (zero for padding rows)
  float qf[S::CPL];
  if (j < m) {
    const uint16_t* qrow = a.q + (((size_t)b * m + j) * a.H + h) * D + g * S::CPL;
#pragma unroll
    for (int c = 0; c < S::CPL; c += 8) {
      const uint4 w = ld16(qrow + c);
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        qf[c + 2 * k] = lo_h(ws[k]) * a.qscale;
        qf[c + 2 * k + 1] = hi_h(ws[k]) * a.qscale;
      }
    }
  } else {
#pragma unroll
    for (int c = 0; c < S::CPL; ++c) qf[c] = 0.f;
  }

  float m_run = -INFINITY, l_run = 0.f, beta = 0.f;
  f32x4 O[S::RT];
#pragma unroll
  for (int rt = 0; rt < S::RT; ++rt) O[rt] = f32x4{0.f, 0.f, 0.f, 0.f};

  constexpr int KB = D / 8;  // key-row bytes per lane group
  for (int gi = g0; gi < g1; ++gi) {
    const uint8_t* ukg = a.uk + (bh * a.T + (size_t)gi * kGroup) * (D / 2);
    const uint8_t* lkg = a.lk + (bh * a.T + (size_t)gi * kGroup) * (D / 2);
    const uint8_t* uvg = a.uv + ((bh * a.NG + gi) * D) * (kGroup / 2);
    const uint8_t* lvg = a.lv + ((bh * a.NG + gi) * D) * (kGroup / 2);
    uint32_t ku[8][S::KK], kl[8][S::KK];
#pragma unroll
    for (int tau = 0; tau < 8; ++tau) {
      const size_t rowoff = (size_t)tile_row_token(tau, j) * (D / 2) + g * KB;
      if constexpr (S::KK == 4) {
        const uint4 u = ld16(ukg + rowoff), l = ld16(lkg + rowoff);
        ku[tau][0] = u.x; ku[tau][1] = u.y; ku[tau][2] = u.z; ku[tau][3] = u.w;
        kl[tau][0] = l.x; kl[tau][1] = l.y; kl[tau][2] = l.z; kl[tau][3] = l.w;
      } else {
        const uint2 u = *reinterpret_cast<const uint2*>(ukg + rowoff);
        const uint2 l = *reinterpret_cast<const uint2*>(lkg + rowoff);
        ku[tau][0] = u.x; ku[tau][1] = u.y;
        kl[tau][0] = l.x; kl[tau][1] = l.y;
      }
    }
    uint4 vu[S::RT], vl[S::RT];
#pragma unroll
    for (int rt = 0; rt < S::RT; ++rt) {
      const size_t off = (size_t)(16 * rt + j) * (kGroup / 2) + g * 16;
      vu[rt] = ld16(uvg + off);
      vl[rt] = ld16(lvg + off);
    }
    float4 km = make_float4(0.f, 0.f, 0.f, 0.f);
    if (lane < D / 2)
      km = *reinterpret_cast<const float4*>(a.kmeta + (((bh * a.NG + gi) * D) + 2 * lane) * 2);
    const float4 vm = *reinterpret_cast<const float4*>(a.vmeta + ((bh * a.T) + (size_t)gi * kGroup + 2 * lane) * 2);

    __syncthreads();
    if (lane < D / 2) {
      L.km[2 * lane] = make_float2(km.x, km.y);
      L.km[2 * lane + 1] = make_float2(km.z, km.w);
    }
    L.vm[2 * lane] = make_float2(vm.x, vm.x * (128.f - vm.y));
    L.vm[2 * lane + 1] = make_float2(vm.z, vm.z * (128.f - vm.w));
    __syncthreads();

    // q' = q * s as fp16 hi + lo (B operands) and bias = sum_d (1024 (q'h + q'l)_d + q'_d z_d)
    f16x8 Bq[S::KK], Bql[S::KK];
    float bias = 0.f;
#pragma unroll
    for (int kk = 0; kk < S::KK; ++kk) {
      f16 qh[8], ql[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int c = 8 * kk + e;
        const float2 sz = L.km[g * S::CPL + c];
        const float qp = qf[c] * sz.x;
        split_f16(qp, qh[e], ql[e]);
        bias += 1024.f * ((float)qh[e] + (float)ql[e]) + qp * sz.y;
      }
      Bq[kk] = f16x8{qh[0], qh[2], qh[4], qh[6], qh[1], qh[3], qh[5], qh[7]};
      Bql[kk] = f16x8{ql[0], ql[2], ql[4], ql[6], ql[1], ql[3], ql[5], ql[7]};
    }
    bias += __shfl_xor(bias, 16);
    bias += __shfl_xor(bias, 32);

    f32x4 St[8];
#pragma unroll
    for (int tau = 0; tau < 8; ++tau) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < S::KK; ++kk) {
        const f16x8 A = codes_f16(ku[tau][kk], kl[tau][kk]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, Bq[kk], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, Bql[kk], acc, 0, 0, 0);
      }
      St[tau] = acc - bias;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int tau = 0; tau < 8; ++tau)
      mx = fmaxf(mx, fmaxf(fmaxf(St[tau][0], St[tau][1]), fmaxf(St[tau][2], St[tau][3])));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = exp2f(m_run - m_new);
    m_run = m_new;
    l_run *= alpha;
    beta *= alpha;
#pragma unroll
    for (int rt = 0; rt < S::RT; ++rt) O[rt] *= alpha;

    f16 ph[8][4], pl[8][4];
#pragma unroll
    for (int tau = 0; tau < 8; ++tau)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = exp2f(St[tau][i] - m_new);
        const float2 sw = L.vm[32 * g + 8 * (tau >> 1) + 2 * i + (tau & 1)];
        l_run += p;
        beta += p * sw.y;
        split_f16(p * sw.x, ph[tau][i], pl[tau][i]);
      }
    const f16x2 c1152 = {(f16)1152.f, (f16)1152.f};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f16x8 Bp = {ph[2 * q][0], ph[2 * q][1], ph[2 * q][2], ph[2 * q][3],
                        ph[2 * q + 1][0], ph[2 * q + 1][1], ph[2 * q + 1][2], ph[2 * q + 1][3]};
      const f16x8 Bpl = {pl[2 * q][0], pl[2 * q][1], pl[2 * q][2], pl[2 * q][3],
                         pl[2 * q + 1][0], pl[2 * q + 1][1], pl[2 * q + 1][2], pl[2 * q + 1][3]};
#pragma unroll
      for (int rt = 0; rt < S::RT; ++rt) {
        const uint32_t uw = q == 0 ? vu[rt].x : q == 1 ? vu[rt].y : q == 2 ? vu[rt].z : vu[rt].w;
        const uint32_t lw = q == 0 ? vl[rt].x : q == 1 ? vl[rt].y : q == 2 ? vl[rt].z : vl[rt].w;
        f16x8 A = codes_f16(uw, lw);
        const f16x2 a0 = f16x2{A[0], A[1]} - c1152, a1 = f16x2{A[2], A[3]} - c1152;
        const f16x2 a2 = f16x2{A[4], A[5]} - c1152, a3 = f16x2{A[6], A[7]} - c1152;
        A = f16x8{a0.x, a0.y, a1.x, a1.y, a2.x, a2.y, a3.x, a3.y};
        O[rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, Bp, O[rt], 0, 0, 0);
        O[rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, Bpl, O[rt], 0, 0, 0);
      }
    }
  }

  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  beta += __shfl_xor(beta, 16);
  beta += __shfl_xor(beta, 32);
  if (j < m) {
    float* rec = record(a, D, b, h, item, j);
    if (g == 0) {
      rec[0] = m_run;
      rec[1] = l_run;
    }
#pragma unroll
    for (int rt = 0; rt < S::RT; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) rec[kRecPad + 16 * rt + 4 * g + i] = O[rt][i] + beta;
  }
}

// ------------------------------------------------------------------------------------------
// Tail work item: up to 64 fp16 tail tokens, m queries, causal (VALU)
// ------------------------------------------------------------------------------------------

struct TailLds {
  uint32_t q[QS_MAX_QUERIES][64];    // fp16 pairs of the queries (D/2 words used)
  float p[kTailChunk][QS_MAX_QUERIES];
};

template <int D>
__device__ void tail_item(const AttnArgs& a, int b, int h, int chunk, int split, TailLds& L) {
  const int lane = threadIdx.x;
  const int m = a.m;
  const int nt = a.nt[b];
  const int ring = 2 * kGroup;
  const size_t bh = (size_t)b * a.H + h;
  const int t = chunk * kTailChunk + lane;   // logical tail position of this lane's key
  const bool valid = t < nt;
  const int slot = (a.head[b] + t) % ring;

  for (int i = 0; i < m; ++i)
    for (int w = lane; w < D / 2; w += 64)
      L.q[i][w] = reinterpret_cast<const uint32_t*>(a.q + (((size_t)b * m + i) * a.H + h) * D)[w];
  uint32_t kr[D / 2];
  const uint16_t* krow = a.tail_k + (bh * ring + (valid ? slot : 0)) * D;
#pragma unroll
  for (int c = 0; c < D / 2; c += 4) {
    const uint4 w = valid ? ld16(krow + 2 * c) : make_uint4(0, 0, 0, 0);
    kr[c] = w.x; kr[c + 1] = w.y; kr[c + 2] = w.z; kr[c + 3] = w.w;
  }
  __syncthreads();

  for (int i = 0; i < m; ++i) {
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < D / 2; ++c) s = dot2(as_h2(kr[c]), as_h2(L.q[i][c]), s);
    s *= a.qscale;
    const bool vis = valid && t <= nt - m + i;
    if (!vis) s = -INFINITY;
    const float mx = wave_max_from(s, 1);
    const float p = vis ? exp2f(s - mx) : 0.f;
    const float sum = wave_sum_from(p, 1);
    if (lane == 0) {
      float* rec = record(a, D, b, h, split, i);
      rec[0] = mx;
      rec[1] = sum;
    }
    L.p[lane][i] = p;
  }
  __syncthreads();

  // o_i[d] = sum_t p_i[t] v_t[d]; lane owns channels lane*(D/64) ..
  constexpr int CPL = D / 64;
  float acc[QS_MAX_QUERIES][CPL];
#pragma unroll
  for (int i = 0; i < QS_MAX_QUERIES; ++i)
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[i][c] = 0.f;
  const int nvalid = min(kTailChunk, nt - chunk * kTailChunk);
  for (int tt = 0; tt < nvalid; ++tt) {
    const int sl = (a.head[b] + chunk * kTailChunk + tt) % ring;
    const uint16_t* vrow = a.tail_v + (bh * ring + sl) * D;
    float v[CPL];
    if constexpr (CPL == 2) {
      const uint32_t w = reinterpret_cast<const uint32_t*>(vrow)[lane];
      v[0] = lo_h(w);
      v[1] = hi_h(w);
    } else {
      v[0] = (float)__builtin_bit_cast(f16, vrow[lane]);
    }
#pragma unroll
    for (int i = 0; i < QS_MAX_QUERIES; ++i) {
      if (i < m) {
        const float p = L.p[tt][i];
#pragma unroll
        for (int c = 0; c < CPL; ++c) acc[i][c] += p * v[c];
      }
    }
  }
#pragma unroll
  for (int i = 0; i < QS_MAX_QUERIES; ++i) {
    if (i < m) {
      float* rec = record(a, D, b, h, split, i);
#pragma unroll
      for (int c = 0; c < CPL; ++c) rec[kRecPad + CPL * lane + c] = acc[i][c];
    }
  }
}

// ------------------------------------------------------------------------------------------
// Attention launch: blockIdx.x < n_titems_total are tail items, the rest quantized items;
// blockIdx.y is the head.  One wave per block.
// ------------------------------------------------------------------------------------------

__device__ __forceinline__ int find_seq(const int32_t* base, int B, int idx) {
  int b = 0;
  while (b + 1 < B && base[b + 1] <= idx) ++b;
  return b;
}

template <int D, bool DRAFT>
__global__ __launch_bounds__(64) void attn_kernel(const AttnArgs a) {
  __shared__ union {
    DraftLds d;
    VerifyLds v;
    TailLds t;
  } lds;
  const int h = blockIdx.y;
  const int x = blockIdx.x;
  if (x < a.n_titems_total) {
    const int b = find_seq(a.titem_base, a.B, x);
    const int chunk = x - a.titem_base[b];
    const int split = (a.qitem_base[b + 1] - a.qitem_base[b]) + chunk;
    tail_item<D>(a, b, h, chunk, split, lds.t);
  } else {
    const int y = x - a.n_titems_total;
    const int b = find_seq(a.qitem_base, a.B, y);
    const int item = y - a.qitem_base[b];
    if constexpr (DRAFT)
      draft_quant_item<D>(a, b, h, item, lds.d);
    else
      verify_quant_item<D>(a, b, h, item, lds.v);
  }
}

// out[(b, i, h)] = sum_s o_s 2^(m_s - M) / sum_s l_s 2^(m_s - M) over the splits s of (b, h),
// M = max_s m_s.  256 threads: every split's (max, sum) is loaded at once, then the o vectors
// are read as float4 chunks by 256 / (D/4) split phases in parallel and reduced through LDS.
template <int D>
__global__ __launch_bounds__(256) void combine_kernel(const AttnArgs a) {
  constexpr int C4 = D / 4;        // float4 chunks of o
  constexpr int NP = 256 / C4;     // split phases
  constexpr int SMAX = kMaxQuantSplits + kMaxTailItems;
  __shared__ float wsh[SMAX];
  __shared__ float4 part[NP][C4];
  __shared__ float red[2][4];
  const int h = blockIdx.y;
  const int b = blockIdx.x / a.m;
  const int i = blockIdx.x % a.m;
  const int t = threadIdx.x;
  const int lane = t & 63, wv = t >> 6;
  const int ns = (a.qitem_base[b + 1] - a.qitem_base[b]) + (a.titem_base[b + 1] - a.titem_base[b]);

  float mv[2], lv[2];
  float mloc = -INFINITY;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int s = t + 256 * k;
    mv[k] = -INFINITY;
    lv[k] = 0.f;
    if (s < ns) {
      const float* rec = record(a, D, b, h, s, i);
      mv[k] = rec[0];
      lv[k] = rec[1];
    }
    mloc = fmaxf(mloc, mv[k]);
  }
  mloc = wave_max_from(mloc, 1);
  if (lane == 0) red[0][wv] = mloc;
  __syncthreads();
  const float M = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));
  float lloc = 0.f;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int s = t + 256 * k;
    if (s < ns) {
      const float w = mv[k] == -INFINITY ? 0.f : exp2f(mv[k] - M);
      wsh[s] = w;
      lloc += w * lv[k];
    }
  }
  lloc = wave_sum_from(lloc, 1);
  if (lane == 0) red[1][wv] = lloc;
  __syncthreads();
  const float L = (red[1][0] + red[1][1]) + (red[1][2] + red[1][3]);

  const int c = t % C4, p = t / C4;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 4
  for (int s = p; s < ns; s += NP) {
    const float4 o = reinterpret_cast<const float4*>(record(a, D, b, h, s, i) + kRecPad)[c];
    const float w = wsh[s];
    acc.x += w * o.x;
    acc.y += w * o.y;
    acc.z += w * o.z;
    acc.w += w * o.w;
  }
  part[p][c] = acc;
  __syncthreads();
  if (t < C4) {
    float4 r = part[0][t];
    for (int q = 1; q < NP; ++q) {
      r.x += part[q][t].x;
      r.y += part[q][t].y;
      r.z += part[q][t].z;
      r.w += part[q][t].w;
    }
    const float inv = 1.f / L;
    float4* out = reinterpret_cast<float4*>(a.out + (((size_t)b * a.m + i) * a.H + h) * D);
    out[t] = make_float4(r.x * inv, r.y * inv, r.z * inv, r.w * inv);
  }
}

// ------------------------------------------------------------------------------------------
// Append: n[b] rows of fp16 K/V per sequence into the ring
// ------------------------------------------------------------------------------------------

template <int D>
__global__ __launch_bounds__(256) void append_kernel(const AppendArgs a) {
  constexpr int CH = D / 8;  // 16-byte chunks per row
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  const int row = idx / CH, c = idx % CH;
  const int h = row % a.H;
  const int i = (row / a.H) % a.n_max;
  const int b = row / (a.H * a.n_max);
  if (b >= a.B || i >= a.n[b]) return;
  const int ring = 2 * kGroup;
  const int slot = (a.head[b] + a.start[b] + i) % ring;
  const size_t src = (((size_t)b * a.n_max + i) * a.H + h) * D + 8 * c;
  const size_t dst = (((size_t)b * a.H + h) * ring + slot) * D + 8 * c;
  *reinterpret_cast<uint4*>(a.tail_k + dst) = ld16(a.k + src);
  *reinterpret_cast<uint4*>(a.tail_v + dst) = ld16(a.v + src);
}

// ------------------------------------------------------------------------------------------
// Flush: quantize and bit-split one G-token ring half of (layer, b, h)
// ------------------------------------------------------------------------------------------
//
// Quantizer, in fp32 and in this order (QuantSpec Guide, quantizer listing):
//   s = max((max - min) / 255, 1e-8);  z = rint(-min / s);  c = clamp(rint(x / s) + z, 0, 255)
// keys: one (s, z) per channel over the G tokens; values: one per token over D channels.

__device__ __forceinline__ float quant_scale(float mn, float mx) {
  float s = (mx - mn) / 255.0f;
  return s < 1e-8f ? 1e-8f : s;
}
__device__ __forceinline__ uint32_t quant_code(float x, float s, float z) {
  float q = rintf(x / s) + z;
  q = q < 0.f ? 0.f : q;
  q = q > 255.f ? 255.f : q;
  return (uint32_t)q;
}

template <int D>
__global__ __launch_bounds__(256) void flush_kernel(const FlushArgs a) {
#pragma clang fp contract(off)
  constexpr int G = kGroup;
  constexpr int RS = D + 2;                 // padded fp16 row stride of the staged tile
  __shared__ f16 tile[G * RS];
  __shared__ uint8_t code[G * D];
  __shared__ float red[2][8][D];
  __shared__ float sz[2][D > G ? D : G];

  const int tid = threadIdx.x;
  const int h = blockIdx.x;
  const int sel = blockIdx.y;
  const int layer = a.layer0 + blockIdx.z;
  const int b = a.b[sel];
  const int grp = a.group[sel];
  const int head = a.head[sel];
  const size_t lbh = ((size_t)layer * a.B + b) * a.H + h;
  const int ring = 2 * G;

  for (int pass = 0; pass < 2; ++pass) {  // 0: keys, 1: values
    const uint16_t* src = (pass == 0 ? a.tail_k : a.tail_v) + (lbh * ring + head) * D;
    for (int c = tid; c < G * D / 8; c += 256) {  // G consecutive ring slots, 16 B per thread
      const int r = c / (D / 8), col = (c % (D / 8)) * 8;
      const uint4 w = ld16(src + (size_t)r * D + col);
      uint32_t* dst = reinterpret_cast<uint32_t*>(&tile[r * RS + col]);
      dst[0] = w.x; dst[1] = w.y; dst[2] = w.z; dst[3] = w.w;
    }
    __syncthreads();
    if (pass == 0) {
      // channel pair p = tid % (D/2); token slice r of NR slices
      constexpr int NP = D / 2, NR = 256 / NP, TPR = G / NR;
      const int p = tid % NP, r = tid / NP;
      float mn0 = INFINITY, mx0 = -INFINITY, mn1 = INFINITY, mx1 = -INFINITY;
      for (int t = r * TPR; t < (r + 1) * TPR; ++t) {
        const float x0 = (float)tile[t * RS + 2 * p], x1 = (float)tile[t * RS + 2 * p + 1];
        mn0 = fminf(mn0, x0); mx0 = fmaxf(mx0, x0);
        mn1 = fminf(mn1, x1); mx1 = fmaxf(mx1, x1);
      }
      red[0][r][2 * p] = mn0; red[0][r][2 * p + 1] = mn1;
      red[1][r][2 * p] = mx0; red[1][r][2 * p + 1] = mx1;
      __syncthreads();
      if (tid < D) {
        float mn = red[0][0][tid], mx = red[1][0][tid];
        for (int k = 1; k < NR; ++k) { mn = fminf(mn, red[0][k][tid]); mx = fmaxf(mx, red[1][k][tid]); }
        const float s = quant_scale(mn, mx);
        const float z = rintf(-mn / s);
        sz[0][tid] = s;
        sz[1][tid] = z;
        float* km = a.kmeta + ((lbh * a.NG + grp) * D + tid) * 2;
        km[0] = s;
        km[1] = z;
      }
      __syncthreads();
      for (int e = tid; e < G * D; e += 256) {
        const int t = e / D, d = e % D;
        code[e] = (uint8_t)quant_code((float)tile[t * RS + d], sz[0][d], sz[1][d]);
      }
      __syncthreads();
      // key planes: token-major rows, byte jb = channel 2jb (bits 0-3) | 2jb+1 (bits 4-7)
      uint8_t* uk = a.uk + (lbh * a.T + (size_t)grp * G) * (D / 2);
      uint8_t* lk = a.lk + (lbh * a.T + (size_t)grp * G) * (D / 2);
      for (int c = tid; c < G * D / 32; c += 256) {  // 16 output bytes = 32 codes of one row
        const int t = c / (D / 32), c0 = (c % (D / 32)) * 32;
        uint32_t u[4], l[4];
        for (int k = 0; k < 4; ++k) {
          u[k] = 0; l[k] = 0;
          for (int e = 0; e < 8; ++e) {
            const uint32_t cc = code[t * D + c0 + 8 * k + e];
            u[k] |= (cc >> 4) << (4 * e);
            l[k] |= (cc & 15u) << (4 * e);
          }
        }
        const size_t o = (size_t)t * (D / 2) + c0 / 2;
        *reinterpret_cast<uint4*>(uk + o) = make_uint4(u[0], u[1], u[2], u[3]);
        *reinterpret_cast<uint4*>(lk + o) = make_uint4(l[0], l[1], l[2], l[3]);
      }
    } else {
      // token t = tid / 2, half of its channels each
      const int t = tid >> 1, hf = tid & 1;
      float mn = INFINITY, mx = -INFINITY;
      for (int d = hf * (D / 2); d < (hf + 1) * (D / 2); ++d) {
        const float x = (float)tile[t * RS + d];
        mn = fminf(mn, x);
        mx = fmaxf(mx, x);
      }
      mn = fminf(mn, __shfl_xor(mn, 1));
      mx = fmaxf(mx, __shfl_xor(mx, 1));
      const float s = quant_scale(mn, mx);
      const float z = rintf(-mn / s);
      if (hf == 0) {
        float* vm = a.vmeta + (lbh * a.T + (size_t)grp * G + t) * 2;
        vm[0] = s;
        vm[1] = z;
      }
      for (int d = hf * (D / 2); d < (hf + 1) * (D / 2); ++d)
        code[t * D + d] = (uint8_t)quant_code((float)tile[t * RS + d], s, z);
      __syncthreads();
      // value planes: channel-major rows of G/2 bytes, byte jb = token 2jb | 2jb+1
      uint8_t* uv = a.uv + ((lbh * a.NG + grp) * D) * (G / 2);
      uint8_t* lv = a.lv + ((lbh * a.NG + grp) * D) * (G / 2);
      for (int c = tid; c < D * G / 32; c += 256) {  // 16 output bytes = 32 tokens of one channel
        const int d = c / (G / 32), t0 = (c % (G / 32)) * 32;
        uint32_t u[4], l[4];
        for (int k = 0; k < 4; ++k) {
          u[k] = 0; l[k] = 0;
          for (int e = 0; e < 8; ++e) {
            const uint32_t cc = code[(t0 + 8 * k + e) * D + d];
            u[k] |= (cc >> 4) << (4 * e);
            l[k] |= (cc & 15u) << (4 * e);
          }
        }
        const size_t o = (size_t)d * (G / 2) + t0 / 2;
        *reinterpret_cast<uint4*>(uv + o) = make_uint4(u[0], u[1], u[2], u[3]);
        *reinterpret_cast<uint4*>(lv + o) = make_uint4(l[0], l[1], l[2], l[3]);
      }
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------------------------------
// Launchers (called by the C ABI in qs_api.cpp)
// ------------------------------------------------------------------------------------------

hipError_t launch_append(const AppendArgs& a, int D, hipStream_t st) {
  const long long rows = (long long)a.B * a.n_max * a.H;
  const long long threads = rows * (D / 8);
  if (threads == 0) return hipSuccess;
  const dim3 grid((unsigned)((threads + 255) / 256));
  if (D == 128) hipLaunchKernelGGL(append_kernel<128>, grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL(append_kernel<64>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_flush(const FlushArgs& a, int D, int n_layers, hipStream_t st) {
  const dim3 grid(a.H, a.n_sel, n_layers);
  if (D == 128) hipLaunchKernelGGL(flush_kernel<128>, grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL(flush_kernel<64>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_attention(const AttnArgs& a, int D, bool draft, hipStream_t st) {
  const dim3 grid(a.n_titems_total + a.n_qitems_total, a.H);
  if (D == 128) {
    if (draft) hipLaunchKernelGGL((attn_kernel<128, true>), grid, dim3(64), 0, st, a);
    else hipLaunchKernelGGL((attn_kernel<128, false>), grid, dim3(64), 0, st, a);
  } else {
    if (draft) hipLaunchKernelGGL((attn_kernel<64, true>), grid, dim3(64), 0, st, a);
    else hipLaunchKernelGGL((attn_kernel<64, false>), grid, dim3(64), 0, st, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 cgrid(a.B * a.m, a.H);
  if (D == 128) hipLaunchKernelGGL(combine_kernel<128>, cgrid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL(combine_kernel<64>, cgrid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace qs
