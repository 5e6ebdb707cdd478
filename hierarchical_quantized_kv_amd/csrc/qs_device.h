#pragma once

// qs_device.h -- device code of the hierarchical INT8 KV cache for gfx950 (MI355X): the kernel
// templates and their helpers.  Each launcher translation unit (qs_attn_*.hip, qs_quant.hip)
// instantiates the kernels it launches, so the units compile in parallel.
//
//
// Kernels (one wave64 per work item unless noted):
//   append_kernel   fp16 rows -> tail ring slots
//   flush_kernel    oldest G-token ring half -> per-group asymmetric 8-bit codes, split into the
//                   upper / lower nibble planes, plus (scale, zero-point) metadata; one wave per
//                   32-channel key slice or 32-token value slice
//   attn_kernel     split-K attention work items of one pass:
//                     draft quantized item : upper key / value planes only, VALU (signed
//                                            4-bit integer dot products)
//                     verify quantized item: both planes, MFMA 16x16x32 f16
//                     tail item            : up to 64 fp16 tail tokens, VALU, causal mask
//                   each writes one log-sum-exp partial (max, sum, o[D]) per query
//   combine_kernel  merges the partials of one (sequence, query, head)
// The attention, combine and flush kernels number their workgroups XCD-contiguously (see
// xcd_contiguous_block).
//
// Sources: QuantSpec Guide (aifetchly), "Hierarchical Quantizer with Bit-Packing" listing
// (quantizer, unpack_for_draft, unpack_for_target); Pith review of arXiv:2502.10424, "What carries
// the argument" and Fig. 3 (C8 = 16*C_U + C_L, shared scale and zero-point), Fig. 7 and reference
// [128] (keys channel-wise, values token-wise; Flash-Decoding-compatible split softmax).
//
// Arithmetic of the quantized parts.  With per-channel key metadata (s_d, z_d) of the group and
// the query pre-scaled by sm_scale*log2(e):
//   draft score  = sum_d q_d s_d (16 U_d + off - z_d)
//                = 16 sum_d q'_d (U_d - 8) + sum_d q'_d (128 + off - z_d)
//   verify score = sum_d q'_d C8_d - sum_d q'_d z_d,                 q'_d = q_d s_d
// and with per-token value metadata (s_t, z_t) and softmax weights p_t:
//   draft  o_d = 16 sum_t p'_t (U_td - 8) + sum_t p_t s_t (128 + off - z_t)
//   verify o_d =    sum_t p'_t (C8_td - 128) + sum_t p_t s_t (128 - z_t),   p'_t = p_t s_t
// The first sums of the draft run as signed 4-bit integer dot products against fixed-point
// digits of q' and p'; those of verify on MFMA with fp16 operands built from the codes with the
// magic-number trick (0x6400 | n is the fp16 value 1024 + n).  The second (bias) sums stay in
// fp32, which keeps degenerate groups (scale clamped to 1e-8, huge zero-point) exact.
// With fp16 metadata (scale s, offset b = -s z) a code stands for s C + b: the bias sums take
// s (128 + off) + b and 128 s + b per token, and -q b per channel, in place of the (s, z) forms.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <atomic>
#include <type_traits>

#include "qs_args.h"

namespace qs {

typedef _Float16 f16;
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));


__device__ __forceinline__ f16x2 as_h2(uint32_t x) { return __builtin_bit_cast(f16x2, x); }
__device__ __forceinline__ float dot2(f16x2 a, f16x2 b, float c) {
  return __builtin_amdgcn_fdot2(a, b, c, false);
}
// Power of two f such that every verify value weight of a group, p_t s_t <= smax (p_t <= 1),
// scaled by f stays below 2^14: the fp16 hi/lo weights then keep full relative precision
// instead of falling into the fp16 subnormal range for small softmax probabilities.
__device__ __forceinline__ float weight_scale(float smax) {
  int e;
  frexpf(smax, &e);  // smax < 2^e
  return ldexpf(1.f, 14 - e);
}

// 2^x with the hardware instruction (results below 2^-126 flush to zero).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
// Buffer loads: a wave-uniform resource (base address and byte range in SGPRs) plus a per-lane
// 32-bit offset, with the streaming (non-temporal) cache policy.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
constexpr int kNt = 2;
__device__ __forceinline__ uint4 bld16(rsrc_t r, uint32_t voff, uint32_t soff) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kNt);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 bld8(rsrc_t r, uint32_t voff, uint32_t soff) {
  const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, kNt);
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ float4 bldf4(rsrc_t r, uint32_t voff, uint32_t soff) {
  const uint4 v = bld16(r, voff, soff);
  return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z),
                     __uint_as_float(v.w));
}

// Layout of the upper planes (kFmtNibble / kFmtSplit4 / kFmtSplit2, qs_args.h), a template
// argument of the attention kernels.  In a split plane row each 32-bit word covers 16 entries 16w .. 16w+15 (channels of a key row,
// tokens of a value row); nibble e of the top-plane word holds C_T(16w + e) in its upper two
// bits and C_T(16w + 8 + e) in its lower two, the middle-plane word C_M(16w + e) in its lower
// two bits and C_M(16w + 8 + e) in its upper two.  Then the upper-nibble words of entries
// 16w + 0..7 and 16w + 8..15 are bitfield selects: (T & 0xCC..) | (M & 0x33..) and
// ((T << 2) & 0xCC..) | ((M >> 2) & 0x33..).
// The streams of one (sequence, head) of a layer (mk / mv: the middle planes of the split
// layout, in which uk / uv address the top planes).
struct Streams {
  rsrc_t uk, lk, uv, lv, km, vm, mk, mv;
};
template <bool M16, int FMT = kFmtNibble, class Args>
__device__ __forceinline__ Streams make_streams(const Args& a, size_t bh, int D) {
  const uint32_t plane = (uint32_t)a.T * (uint32_t)(D / 2);  // bytes of one plane per (b, h)
  constexpr uint32_t mb = M16 ? 4 : 8;                       // bytes of one metadata pair
  Streams st;
  if constexpr (FMT == kFmtNibble) {
    st.uk = make_rsrc(a.uk + bh * plane, plane);
    st.uv = make_rsrc(a.uv + bh * plane, plane);
    st.mk = st.uk;
    st.mv = st.uv;
  } else {
    st.uk = make_rsrc(a.uk + bh * plane, plane / 2);
    st.mk = make_rsrc(a.uk + bh * plane + plane / 2, plane / 2);
    st.uv = make_rsrc(a.uv + bh * plane, plane / 2);
    st.mv = make_rsrc(a.uv + bh * plane + plane / 2, plane / 2);
  }
  st.lk = make_rsrc(a.lk + bh * plane, plane);
  st.lv = make_rsrc(a.lv + bh * plane, plane);
  st.km = make_rsrc(a.kmeta + bh * (size_t)a.NG * D * mb, (uint32_t)a.NG * D * mb);
  st.vm = make_rsrc(a.vmeta + bh * (size_t)a.T * mb, (uint32_t)a.T * mb);
  return st;
}

// Upper-nibble words of the 16 entries of a split-layout word pair (top t, middle m): entries
// 0..7 and 8..15 (see kFmtSplit4).
__device__ __forceinline__ uint32_t bfi(uint32_t mask, uint32_t a, uint32_t b) {
  return (a & mask) | (b & ~mask);
}
__device__ __forceinline__ uint2 split_nibbles(uint32_t t, uint32_t m) {
  return make_uint2(bfi(0xCCCCCCCCu, t, m), bfi(0xCCCCCCCCu, t << 2, m >> 2));
}
// 2-bit draft words of a top-plane word: nibble e = C_T (0..3, a non-negative signed nibble)
// of entries 0..7 and of entries 8..15.
__device__ __forceinline__ uint2 top2_values(uint32_t t) {
  return make_uint2((t >> 2) & 0x33333333u, t & 0x33333333u);
}
__device__ __forceinline__ uint32_t bld4(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, kNt);
}

__device__ __forceinline__ float lo_h(uint32_t x) { return (float)as_h2(x).x; }
__device__ __forceinline__ float hi_h(uint32_t x) { return (float)as_h2(x).y; }

// Metadata of two channels (keys) or two tokens (values) as one lane loads it: fp32 (s0, z0,
// s1, z1), or with M16 the fp16 pairs (s0, b0), (s1, b1) in two words, where b = -s z.  meta4
// gives (s0, x0, s1, x1) with x the zero-point (fp32) or the offset (fp16): a code C stands for
// s (C - x) or s C + x.
template <bool M16>
using MetaT = typename std::conditional<M16, uint2, float4>::type;
template <bool M16>  // pairs first + 2 lane, first + 2 lane + 1
__device__ __forceinline__ MetaT<M16> load_meta(rsrc_t r, uint32_t first) {
  const int lane = threadIdx.x;
  if constexpr (M16) return bld8(r, lane * 8, first * 4);
  else return bldf4(r, lane * 16, first * 8);
}
template <bool M16>
__device__ __forceinline__ float4 meta4(const MetaT<M16>& m) {
  if constexpr (M16) return make_float4(lo_h(m.x), hi_h(m.x), lo_h(m.y), hi_h(m.y));
  else return m;
}
template <bool M16>
__device__ __forceinline__ MetaT<M16> make_meta_zero() {
  if constexpr (M16) return make_uint2(0u, 0u);
  else return make_float4(0.f, 0.f, 0.f, 0.f);
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

// Cross-lane steps with DPP (no LDS round trip): quad_perm swaps inside groups of four lanes,
// the mirrors inside half rows (8 lanes) and rows (16 lanes); readlane reads the four rows.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;
constexpr int kDppRor8 = 0x128;       // row_ror:8: lane j of a row reads lane j ^ 8
__device__ __forceinline__ float lane_read(float x, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}
// Sum / max over all 64 lanes; every lane gets the result.
__device__ __forceinline__ float wave_sum_all(float x) {
  x += dpp<kDppXor1>(x);
  x += dpp<kDppXor2>(x);
  x += dpp<kDppHalfMirror>(x);
  x += dpp<kDppMirror>(x);
  return (lane_read(x, 0) + lane_read(x, 16)) + (lane_read(x, 32) + lane_read(x, 48));
}
__device__ __forceinline__ float wave_max_all(float x) {
  x = fmaxf(x, dpp<kDppXor1>(x));
  x = fmaxf(x, dpp<kDppXor2>(x));
  x = fmaxf(x, dpp<kDppHalfMirror>(x));
  x = fmaxf(x, dpp<kDppMirror>(x));
  return fmaxf(fmaxf(lane_read(x, 0), lane_read(x, 16)), fmaxf(lane_read(x, 32), lane_read(x, 48)));
}

__device__ __forceinline__ float wave_max_from(float x, int from) {
  for (int o = from; o < 64; o <<= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum_from(float x, int from) {
  for (int o = from; o < 64; o <<= 1) x += __shfl_xor(x, o);
  return x;
}

// Device mode: nt of sequence b after the pending operations, each applied only if it passes
// the check of the host verb (an append within the 2G ring, a rollback count in 0 .. nt);
// *bad (if given) receives the error bits of the ones that fail.
__device__ __forceinline__ int apply_pending(int nt, const Pending& p, int b, int32_t* bad) {
  int32_t e = 0;
  for (int k = 0; k < p.count; ++k) {
    const PendingOp& o = p.op[k];
    if (o.kind == 0) {
      if (nt + o.n <= 2 * kGroup) nt += o.n;
      else e |= kDevErrAppend;
    } else {
      const int d = o.n - (o.sub ? o.sub[b] : 0);
      if (d >= 0 && d <= nt) nt -= d;
      else e |= kDevErrRollback;
    }
  }
  if (bad) *bad = e;
  return nt;
}

// Counters of sequence b: the by-value copies, or in device mode this layer's state entries
// (nt with the pending operations applied).
template <class Args>
__device__ __forceinline__ int seq_nq(const Args& a, int b) {
  if constexpr (Args::kMode == kModeDev) return a.dev.dstate[kStateInts * b];
  else return a.nq[b];
}
template <class Args>
__device__ __forceinline__ int seq_nt(const Args& a, int b) {
  if constexpr (Args::kMode == kModeDev) return apply_pending(a.dev.dstate[kStateInts * b + 1], a.dev.pend, b, nullptr);
  else return a.nt[b];
}
template <class Args>
__device__ __forceinline__ int seq_head(const Args& a, int b) {
  if constexpr (Args::kMode == kModeDev) return a.dev.dstate[kStateInts * b + 2];
  else return a.head[b];
}

// Query column c of (b, h): its row in q and out ([B][m][H][D]; with grouped queries column
// c = i gq + r is query token i of query head h gq + r, [B][mt][hq][D]), and its query token
// (for the causal mask among the tail tokens) out of how many.
template <class Args>
__device__ __forceinline__ size_t qrow(const Args& a, int b, int h, int c) {
  if constexpr (Args::kMode == kModeGqa)
    return ((size_t)b * a.mt + c / a.gq) * a.hq + (size_t)h * a.gq + c % a.gq;
  else
    return ((size_t)b * a.m + c) * a.H + h;
}
template <class Args>
__device__ __forceinline__ int col_token(const Args& a, int c) {
  if constexpr (Args::kMode == kModeGqa) return c / a.gq;
  else return c;
}
template <class Args>
__device__ __forceinline__ int n_tokens(const Args& a) {
  if constexpr (Args::kMode == kModeGqa) return a.mt;
  else return a.m;
}

// Record of split `split`, query `i` of (b, h).
template <class Args>
__device__ __forceinline__ float* record(const Args& a, int D, int b, int h, int split, int i) {
  return a.work + ((((size_t)b * a.H + h) * a.S + split) * a.m + i) * (size_t)(D + kRecPad);
}

// Group assignment of the quantized workers of (b, h): worker w of W takes groups w, w + W,
// w + 2W, ...  At every step the W workers of a head read one contiguous run of W groups, so the
// plane traffic of the whole call spreads evenly over the HBM channels (contiguous per-worker
// chunks were measured to leave some waves twice as slow as others).
struct GroupStride {
  int first, step, ng;
};
template <class Args>
__device__ __forceinline__ GroupStride worker_groups(const Args& a, int b, int item) {
  return GroupStride{item, a.qitem_base[b + 1] - a.qitem_base[b], seq_nq(a, b) / kGroup};
}

// The waves that share a SIMD issue oldest first, so with equal work the oldest finishes far
// ahead of the youngest, and the SIMD spends the end of the call with a single wave and little
// memory traffic in flight.  Each worker therefore sets its issue priority from the fraction of
// its groups still to do (four levels): a worker that falls behind keeps precedence until the
// others have caught up.
__device__ __forceinline__ void pace(int remaining, int total) {
  const int q = (4 * remaining + total - 1) / total;  // 1 .. 4
  if (q >= 4)
    __builtin_amdgcn_s_setprio(3);
  else if (q == 3)
    __builtin_amdgcn_s_setprio(2);
  else if (q == 2)
    __builtin_amdgcn_s_setprio(1);
  else
    __builtin_amdgcn_s_setprio(0);
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

// Draft arithmetic in integers.  An upper nibble U is taken as the signed 4-bit u = U - 8
// (the nibble XOR 8), and a weight x (q' for keys, p' for values) as a fixed-point integer
// X = round(x / unit) with |X| < 2^22, written in six signed base-16 digits c_j in [-8, 7]
// (X = sum_j 16^j c_j: the nibbles of X + 0x888888, each XOR 8).  Then
//   sum_e x_e u_e = unit * sum_j 16^j sum_e c_j,e u_e,
// and every inner sum over the 8 nibbles of a 32-bit plane word is one v_dot8_i32_i4, exact in
// int32.  The unit is a power of two chosen per group from the largest weight, so the products
// lose only the rounding of x to 22 bits relative to that largest weight.
constexpr int kDigits = 6;
constexpr uint32_t kDigitBias = 0x888888u;  // 8 in each of the six digit positions
constexpr uint32_t kNibbleBias = 0x88888888u;

struct DraftLds {
  uint32_t qd[kDigits][16];       // key weights q': digit j of channels 8w .. 8w+7 in word w
  uint32_t pd[kDigits][kGroup / 8];  // value weights p' = p s: digit j of tokens 8w .. 8w+7
  float2 vm[kGroup];              // (s_t, s_t * (128 + off - z_t))
};

// Digit bytes of two fixed-point weights a (low nibbles) and b (high nibbles): byte k of `even`
// is digit 2k, byte k of `odd` digit 2k+1, both already XOR 8.
__device__ __forceinline__ void digit_bytes(int xa, int xb, uint32_t& even, uint32_t& odd) {
  const uint32_t a = (uint32_t)xa + kDigitBias, b = (uint32_t)xb + kDigitBias;
  even = ((a & 0x0F0F0Fu) | ((b & 0x0F0F0Fu) << 4)) ^ kDigitBias;
  odd = (((a >> 4) & 0x0F0F0Fu) | (((b >> 4) & 0x0F0F0Fu) << 4)) ^ kDigitBias;
}

// sum over 4 signed-nibble words u[] (32 nibbles, each the signed 4-bit value of one entry) of
// the digit-weighted signed dot products, as a float in units of the fixed-point weights:
// sum_j 16^j sum_k dot8(d[j].k, u[k]) over the ND lowest digit planes.  Six planes of signed
// nibbles run as two Horner chains (digits 5..3 and 2..0; |chain| <= 2048 * 273 fits int32);
// five planes of 2-bit values as one.
template <int ND = kDigits>
__device__ __forceinline__ float digit_dot(const uint4 (&d)[kDigits], uint4 w) {
  static_assert(ND == 5 || ND == 6, "five or six digit planes");
  const int u[4] = {(int)w.x, (int)w.y, (int)w.z, (int)w.w};
  auto plane = [&](int j, int acc) {
    acc = __builtin_amdgcn_sdot8((int)d[j].x, u[0], acc, false);
    acc = __builtin_amdgcn_sdot8((int)d[j].y, u[1], acc, false);
    acc = __builtin_amdgcn_sdot8((int)d[j].z, u[2], acc, false);
    return __builtin_amdgcn_sdot8((int)d[j].w, u[3], acc, false);
  };
  if constexpr (ND == 5) {
    // entries in 0..3 (the 2-bit draft): |plane| <= 768, so one chain stays below 768 * 69905
    int acc = plane(4, 0);
    acc = plane(3, acc << 4);
    acc = plane(2, acc << 4);
    acc = plane(1, acc << 4);
    acc = plane(0, acc << 4);
    return (float)acc;
  } else {
    int hi = plane(5, 0);
    hi = plane(4, hi << 4);
    hi = plane(3, hi << 4);
    int lo = plane(2, 0);
    lo = plane(1, lo << 4);
    lo = plane(0, lo << 4);
    return fmaf((float)hi, 4096.f, (float)lo);
  }
}

// Power-of-two fixed-point unit for weights up to xmax: |x| / unit < 2^BITS (22 for six
// digits; 18 for five, whose top digit then stays zero).
template <int BITS = 22>
__device__ __forceinline__ void fixed_unit(float xmax, float& inv_unit, float& unit) {
  int e;
  frexpf(xmax, &e);  // xmax < 2^e (e = 0 for xmax = 0)
  inv_unit = ldexpf(1.f, BITS - e);
  unit = ldexpf(1.f, e - BITS);
}

// Planes and metadata of one group, as loaded by one lane: per key load 32 channels of one
// token row, per value load 32 tokens of one channel row (16 bytes of the nibble plane, or 8
// bytes of each 2-bit plane).
template <int FMT>
using DraftW = typename std::conditional<FMT == kFmtNibble, uint4, uint2>::type;
template <int D, bool M16, int FMT>
struct DraftBuf {
  using W = DraftW<FMT>;
  static constexpr int KM = FMT == kFmtSplit4 ? DraftShape<D>::KIT : 1;  // middle-plane words
  static constexpr int VM = FMT == kFmtSplit4 ? DraftShape<D>::VIT : 1;
  W k[DraftShape<D>::KIT];   // upper nibble plane, or top plane
  W v[DraftShape<D>::VIT];
  uint2 k2[KM];              // kFmtSplit4: middle plane
  uint2 v2[VM];
  MetaT<M16> km;  // key metadata of channels 2*lane, 2*lane+1
  MetaT<M16> vm;  // value metadata of tokens 2*lane, 2*lane+1
};

// The signed-nibble words digit_dot takes (nibble = upper nibble - 8; for the 2-bit draft the
// top bits C_T in 0..3) of one load: its 32 entries in order, 8 per word.
template <int FMT>
__device__ __forceinline__ uint4 signed_words(const DraftW<FMT>& x, uint2 mid) {
  if constexpr (FMT == kFmtNibble) {
    return make_uint4(x.x ^ kNibbleBias, x.y ^ kNibbleBias, x.z ^ kNibbleBias, x.w ^ kNibbleBias);
  } else if constexpr (FMT == kFmtSplit4) {
    const uint2 a = split_nibbles(x.x ^ 0xAAAAAAAAu, mid.x), b = split_nibbles(x.y ^ 0xAAAAAAAAu, mid.y);
    return make_uint4(a.x, a.y, b.x, b.y);
  } else {
    const uint2 a = top2_values(x.x), b = top2_values(x.y);
    return make_uint4(a.x, a.y, b.x, b.y);
  }
}

template <int D, int FMT, bool M16>
__device__ __forceinline__ void draft_load_k(const Streams& sm, int g, DraftBuf<D, M16, FMT>& buf) {
  using S = DraftShape<D>;
  const int lane = threadIdx.x;
  if constexpr (FMT == kFmtNibble) {
    const uint32_t voff = (lane / S::KL) * (D / 2) + (lane % S::KL) * 16;
    const uint32_t soff = (uint32_t)g * kGroup * (D / 2);
#pragma unroll
    for (int it = 0; it < S::KIT; ++it)  // key rows it*TPI .. : 1 KB apart
      buf.k[it] = bld16(sm.uk, voff + (it & 3) * 1024, soff + (it >> 2) * 4096);
  } else {
    const uint32_t voff = (lane / S::KL) * (D / 4) + (lane % S::KL) * 8;
    const uint32_t soff = (uint32_t)g * kGroup * (D / 4);
#pragma unroll
    for (int it = 0; it < S::KIT; ++it) {
      buf.k[it] = bld8(sm.uk, voff + it * S::TPI * (D / 4), soff);
      if constexpr (FMT == kFmtSplit4) buf.k2[it] = bld8(sm.mk, voff + it * S::TPI * (D / 4), soff);
    }
  }
}
template <int D, int FMT, bool M16>
__device__ __forceinline__ void draft_load_meta(const Streams& sm, int g, DraftBuf<D, M16, FMT>& buf) {
  const int lane = threadIdx.x;
  // lanes >= D/2 hold no channels.  At D = 64 zeroing their registers here makes the wave wait
  // for all of its loads once per group, which measured faster at 128k than masking at the use.
  buf.km = load_meta<M16>(sm.km, (uint32_t)g * D);
  if (lane >= D / 2) buf.km = make_meta_zero<M16>();
  buf.vm = load_meta<M16>(sm.vm, (uint32_t)g * kGroup);
}
template <int D, int FMT, bool M16>
__device__ __forceinline__ void draft_load_v(const Streams& sm, int g, DraftBuf<D, M16, FMT>& buf) {
  using S = DraftShape<D>;
  const int lane = threadIdx.x;
  const int vr = lane & 3, vd = lane >> 2;
  if constexpr (FMT == kFmtNibble) {
    const uint32_t voff = (vr >> 1) * (D * kGroup / 4) + vd * (kGroup / 4) + (vr & 1) * 16;
    const uint32_t soff = (uint32_t)g * D * (kGroup / 2);
#pragma unroll
    for (int i = 0; i < S::VIT; ++i) buf.v[i] = bld16(sm.uv, voff + i * 16 * (kGroup / 4), soff);
  } else {
    const uint32_t voff = (vr >> 1) * (D * kGroup / 8) + vd * (kGroup / 8) + (vr & 1) * 8;
    const uint32_t soff = (uint32_t)g * D * (kGroup / 4);
#pragma unroll
    for (int i = 0; i < S::VIT; ++i) {
      buf.v[i] = bld8(sm.uv, voff + i * 16 * (kGroup / 8), soff);
      if constexpr (FMT == kFmtSplit4) buf.v2[i] = bld8(sm.mv, voff + i * 16 * (kGroup / 8), soff);
    }
  }
}

// Running softmax state of a draft work item (per lane).
template <int D>
struct DraftAcc {
  float m_run, l_run, beta;
  float o[DraftShape<D>::VIT];
};

// One group: scores of its 128 keys from the upper key plane, online-softmax update, and the
// weighted sum of its upper value plane.
// With PF the registers of `cur` are refilled with group `gnext` as soon as each part of the
// current group has been consumed, so the next group's loads overlap this group's arithmetic.
// (The prefetch is a template flag rather than a run-time test so that the number of loads in
// flight at every wait is fixed.)
template <int D, bool PF, bool M16, int FMT, class Args>
__device__ __forceinline__ void draft_group(const Args& a, const Streams& sm,
                                            DraftBuf<D, M16, FMT>& cur, int gnext, float q0,
                                            float q1, DraftLds& L, DraftAcc<D>& st) {
  using S = DraftShape<D>;
  const int lane = threadIdx.x;
  const int kc = lane % S::KL, kt = lane / S::KL, vr = lane & 3;
  // 16 U + off - z = 16 u + (128 + off - z); the 2-bit draft: 64 C_T + (4 off - z), its
  // weights on five digits (18 bits: the rounding stays far below the 2-bit codes' steps)
  constexpr bool k2 = FMT == kFmtSplit2;
  constexpr int ND = k2 ? 5 : kDigits;
  constexpr int WB = k2 ? 18 : 22;
  constexpr float kStep = k2 ? 64.f : 16.f;  // weight of one unit of the dot-product entries
  const float c = k2 ? 4.f * a.draft_offset : 128.f + a.draft_offset;

  __syncthreads();  // the previous group's LDS reads are done
  // key weights q' = q s (channels 2 lane, 2 lane + 1) as digit planes; the score bias
  // sum_d q'_d (128 + off - z_d) stays in fp32
  const float4 km = meta4<M16>(cur.km), vm = meta4<M16>(cur.vm);
  const float qa = q0 * km.x, qb = q1 * km.z;  // zero on lanes >= D/2
  // fp16 metadata: s (16 U + off) + b = 16 s (U - 8) + (s (128 + off) + b)
  float bias = M16 ? q0 * fmaf(km.x, c, km.y) + q1 * fmaf(km.z, c, km.w)
                   : qa * (c - km.y) + qb * (c - km.w);
  float qunit, qinv;
  fixed_unit<WB>(wave_max_all(fmaxf(fabsf(qa), fabsf(qb))), qinv, qunit);
  L.vm[2 * lane] = make_float2(vm.x, M16 ? fmaf(vm.x, c, vm.y) : vm.x * (c - vm.y));
  L.vm[2 * lane + 1] = make_float2(vm.z, M16 ? fmaf(vm.z, c, vm.w) : vm.z * (c - vm.w));
  float punit, pinv;  // p' = p s <= max_t s_t
  fixed_unit<WB>(wave_max_all(fmaxf(vm.x, vm.z)), pinv, punit);
  if (lane < D / 2) {
    uint32_t ev, od;
    digit_bytes((int)rintf(qa * qinv), (int)rintf(qb * qinv), ev, od);
    uint8_t* qd = reinterpret_cast<uint8_t*>(&L.qd[0][0]);
#pragma unroll
    for (int j = 0; j < ND; ++j)
      qd[j * 64 + lane] = (uint8_t)(((j & 1) ? od : ev) >> (8 * (j >> 1)));
  }
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (PF) draft_load_meta<D, FMT>(sm, gnext, cur);
  bias = wave_sum_all(bias);
  __syncthreads();

  uint4 dq[kDigits];
#pragma unroll
  for (int j = 0; j < kDigits; ++j) dq[j] = reinterpret_cast<const uint4*>(L.qd[j])[kc];
  const float kscale = kStep * qunit;
  float sc[S::KIT];
#pragma unroll
  for (int it = 0; it < S::KIT; ++it) {
    float p = digit_dot<ND>(dq, signed_words<FMT>(cur.k[it], cur.k2[FMT == kFmtSplit4 ? it : 0]));
    p += dpp<kDppXor1>(p);  // the KL lanes of a key row
    if constexpr (S::KL == 4) p += dpp<kDppXor2>(p);
    sc[it] = fmaf(p, kscale, bias);
  }
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (PF) draft_load_k<D, FMT>(sm, gnext, cur);
  float gmax = sc[0];
#pragma unroll
  for (int it = 1; it < S::KIT; ++it) gmax = fmaxf(gmax, sc[it]);
  gmax = wave_max_all(gmax);
  const float m_new = fmaxf(st.m_run, gmax);
  const float alpha = fast_exp2(st.m_run - m_new);
  st.m_run = m_new;
  st.l_run *= alpha;
  st.beta *= alpha;
  // value weights p' = p s as digit planes.  Token t = it * TPI + kt sits in the KL lanes of its
  // key row; lanes of even rows pair token t with t + 1 (held KL lanes up) into digit bytes, and
  // lane kc of the row writes planes kc * PPL ...
  constexpr int PPL = (ND + S::KL - 1) / S::KL;
  uint8_t* pd = reinterpret_cast<uint8_t*>(&L.pd[0][0]);
#pragma unroll
  for (int it = 0; it < S::KIT; ++it) {
    const int t = it * S::TPI + kt;
    const float p = fast_exp2(sc[it] - m_new);
    const float2 sw = L.vm[t];
    st.l_run += p;
    st.beta += p * sw.y;
    const int x = (int)rintf(p * sw.x * pinv);
    // any lane of the next key row holds that token's weight: half-row mirror (KL = 4) or
    // quad swap (KL = 2), without a round trip through LDS
    const int xn = __builtin_amdgcn_update_dpp(0, x, S::KL == 4 ? kDppHalfMirror : kDppXor2, 0xF, 0xF, false);
    if ((kt & 1) == 0) {
      uint32_t ev, od;
      digit_bytes(x, xn, ev, od);
#pragma unroll
      for (int jj = 0; jj < PPL; ++jj) {
        const int j = kc * PPL + jj;
        if (j < ND) pd[j * (kGroup / 2) + t / 2] = (uint8_t)(((j & 1) ? od : ev) >> (8 * (j >> 1)));
      }
    }
  }
  __syncthreads();

  uint4 dp[kDigits];
#pragma unroll
  for (int j = 0; j < kDigits; ++j) dp[j] = reinterpret_cast<const uint4*>(L.pd[j])[vr];
  const float vscale = kStep * punit;
#pragma unroll
  for (int i = 0; i < S::VIT; ++i) {
    st.o[i] = fmaf(st.o[i], alpha,
                   digit_dot<ND>(dp, signed_words<FMT>(cur.v[i], cur.v2[FMT == kFmtSplit4 ? i : 0])) * vscale);
    __builtin_amdgcn_sched_barrier(0);
  }
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (PF) draft_load_v<D, FMT>(sm, gnext, cur);
}

template <int D, bool M16, int FMT, class Args>
__device__ void draft_quant_item(const Args& a, int b, int h, int item, DraftLds& L) {
  using S = DraftShape<D>;
  const int lane = threadIdx.x;
  const size_t bh = (size_t)b * a.H + h;
  const GroupStride gs = worker_groups(a, b, item);

  float q0 = 0.f, q1 = 0.f;  // channels 2*lane, 2*lane+1 (lanes < D/2), times qscale
  if (lane < D / 2) {
    const uint32_t qq = reinterpret_cast<const uint32_t*>(a.q + bh * D)[lane];
    q0 = lo_h(qq) * a.qscale;
    q1 = hi_h(qq) * a.qscale;
  }
  DraftAcc<D> st;
  st.m_run = -INFINITY;
  st.l_run = 0.f;
  st.beta = 0.f;
#pragma unroll
  for (int i = 0; i < S::VIT; ++i) st.o[i] = 0.f;

  const Streams sm = make_streams<M16, FMT>(a, bh, D);
  DraftBuf<D, M16, FMT> buf;
  if (gs.first < gs.ng) {
    draft_load_k<D, FMT>(sm, gs.first, buf);
    draft_load_meta<D, FMT>(sm, gs.first, buf);
    draft_load_v<D, FMT>(sm, gs.first, buf);
    const int total = (gs.ng - gs.first + gs.step - 1) / gs.step;
    int g = gs.first, done = 0;
    for (; g + gs.step < gs.ng; g += gs.step, ++done) {
      pace(total - done, total);
      draft_group<D, true, M16, FMT>(a, sm, buf, g + gs.step, q0, q1, L, st);
    }
    pace(1, total);
    draft_group<D, false, M16, FMT>(a, sm, buf, -1, q0, q1, L, st);
  }

  // l and beta were accumulated once per key row in each of its KL lanes
  const float l_run = wave_sum_from(st.l_run, S::KL);
  const float beta = wave_sum_from(st.beta, S::KL);
  const int vr = lane & 3, vd = lane >> 2;
  float* rec = record(a, D, b, h, item, 0);
  if (lane == 0) {
    rec[0] = st.m_run;
    rec[1] = l_run;
  }
#pragma unroll
  for (int i = 0; i < S::VIT; ++i) {
    float o = st.o[i];
    o += __shfl_xor(o, 1);
    o += __shfl_xor(o, 2);
    if ((i & 3) == vr) rec[kRecPad + 16 * i + vd] = o + beta;
  }
}

// ------------------------------------------------------------------------------------------
// Verify: quantized work item (both planes, MFMA)
// ------------------------------------------------------------------------------------------
//
// A group of 128 tokens is processed in two halves of 64.  Lane l = 16 g + j (j: query column of
// the MFMA B operand and of the results, g: k-group):
//   S^T tile tau (16 tokens x 16 queries) = sum over D/32 MFMAs of A (key codes) x B (q' slots);
//   row r of tile tau is token 64(tau/4) + 16(r/4) + 8((tau%4)/2) + 2(r%4) + (tau%2), so that in
//   half h lane group g holds exactly tokens 64h + 16g .. 64h + 16g + 15, in the slot order the
//   PV MFMAs need, and reads them as one 8-byte piece of each value-plane row.
//   O^T tile rt (16 channels x 16 queries) += A (value codes - 128) x B (p' of tiles 2q, 2q+1).
// q' = q s and p' = p s enter the MFMAs as fp16 hi + lo pairs; the bias sums stay in fp32.
// With up to kPairMaxQueries query columns (the paired form, PAIR), column j < 8 of a B operand
// holds the hi part of query j and column j + 8 its lo part, so one MFMA takes both: S^T column
// j and j ^ 8 are summed across the row (one DPP step per value), both lanes then hold the same
// score and weight and feed p' hi (j < 8) or lo (j >= 8) to the PV MFMAs, and the O^T columns j
// and j + 8 are summed once at the end.  Half the MFMAs and B registers of the 16-column form.

template <int D>
struct VerifyShape {
  static constexpr int KK = D / 32;   // MFMA k-steps per S^T tile
  static constexpr int CPL = D / 4;   // channels per lane group
  static constexpr int RT = D / 16;   // O^T channel tiles
  static constexpr int KB = D / 8;    // key-row bytes per lane group
};

// MQ: query capacity; PAIR: the paired form (hi and lo in the columns of one B operand)
template <int MQ, bool PAIR>
struct VerifyLdsQ {
  static constexpr int kPlanes = PAIR ? 1 : 2;  // B operand sets: (hi, lo), or both in one
  static constexpr int kCols = PAIR ? 16 : MQ;  // B columns held per k-step and k-group
  float2 qs[MQ][64];                      // queries times qscale, channels (2 lane, 2 lane + 1)
  float2 vm[kGroup];                      // (s_t, s_t * (128 - z_t))
  uint4 bq[kPlanes][4][4 * kCols];        // q' B operands per k-step, k-group and column
  float bias[MQ][64];                     // per-query bias partials of the lanes' channels
};
using VerifyLds = VerifyLdsQ<QS_MAX_QUERIES, false>;
using VerifyLdsPair = VerifyLdsQ<kPairMaxQueries, true>;

__device__ __forceinline__ int vtile_token(int tau, int r) {
  return 64 * (tau >> 2) + 16 * (r >> 2) + 8 * ((tau & 3) >> 1) + 2 * (r & 3) + (tau & 1);
}

template <int D, bool M16>
struct VerifyBuf {
  uint32_t ku[4][VerifyShape<D>::KK], kl[4][VerifyShape<D>::KK];  // 4 key tiles of a half
  uint2 vu[VerifyShape<D>::RT], vl[VerifyShape<D>::RT];            // value codes of a half
  MetaT<M16> km;  // key metadata of channels 2*lane, 2*lane+1
  MetaT<M16> vm;  // value metadata of tokens 2*lane, 2*lane+1
};

// UPPER: only the upper planes are read (the draft pass over grouped queries); the lower
// nibbles are then the draft offset.  FMT: layout of the upper planes (kFmtNibble or
// kFmtSplit4, whose top and middle 2-bit words are turned into the same upper-nibble words).
template <int D, bool UPPER = false, int FMT = kFmtNibble, bool M16>
__device__ __forceinline__ void verify_load_k(const Streams& sm, int gi, int half, VerifyBuf<D, M16>& buf) {
  using S = VerifyShape<D>;
  const int lane = threadIdx.x, j = lane & 15, g = lane >> 4;
  // row of tile 4*half + t for lane row j: 16 (j/4) + 2 (j%4) + 64 half + 8 (t/2) + (t%2)
  const uint32_t row0 = 16 * (j >> 2) + 2 * (j & 3);
  const uint32_t voff = row0 * (D / 2) + g * S::KB;
  const uint32_t soff = ((uint32_t)gi * kGroup + 64 * half) * (D / 2);
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const uint32_t dr = 8 * (t >> 1) + (t & 1);
    const uint32_t o = voff + dr * (D / 2);
    if constexpr (FMT != kFmtNibble) {  // split layout: rows of D/4 bytes, D/16 per lane group
      const uint32_t os = (row0 + dr) * (D / 4) + g * (D / 16);
      const uint32_t ss = ((uint32_t)gi * kGroup + 64 * half) * (D / 4);
      if constexpr (S::KK == 4) {
        const uint2 tw = bld8(sm.uk, os, ss), mw = bld8(sm.mk, os, ss);
        const uint2 a = split_nibbles(tw.x, mw.x), b = split_nibbles(tw.y, mw.y);
        buf.ku[t][0] = a.x; buf.ku[t][1] = a.y; buf.ku[t][2] = b.x; buf.ku[t][3] = b.y;
      } else {
        const uint2 a = split_nibbles(bld4(sm.uk, os, ss), bld4(sm.mk, os, ss));
        buf.ku[t][0] = a.x; buf.ku[t][1] = a.y;
      }
      if constexpr (!UPPER) {
        if constexpr (S::KK == 4) {
          const uint4 l = bld16(sm.lk, o, soff);
          buf.kl[t][0] = l.x; buf.kl[t][1] = l.y; buf.kl[t][2] = l.z; buf.kl[t][3] = l.w;
        } else {
          const uint2 l = bld8(sm.lk, o, soff);
          buf.kl[t][0] = l.x; buf.kl[t][1] = l.y;
        }
      }
    } else if constexpr (S::KK == 4) {
      const uint4 u = bld16(sm.uk, o, soff);
      buf.ku[t][0] = u.x; buf.ku[t][1] = u.y; buf.ku[t][2] = u.z; buf.ku[t][3] = u.w;
      if constexpr (!UPPER) {
        const uint4 l = bld16(sm.lk, o, soff);
        buf.kl[t][0] = l.x; buf.kl[t][1] = l.y; buf.kl[t][2] = l.z; buf.kl[t][3] = l.w;
      }
    } else {
      const uint2 u = bld8(sm.uk, o, soff);
      buf.ku[t][0] = u.x; buf.ku[t][1] = u.y;
      if constexpr (!UPPER) {
        const uint2 l = bld8(sm.lk, o, soff);
        buf.kl[t][0] = l.x; buf.kl[t][1] = l.y;
      }
    }
  }
}

template <int D, bool UPPER = false, int FMT = kFmtNibble, bool M16>
__device__ __forceinline__ void verify_load_v(const Streams& sm, int gi, int half, VerifyBuf<D, M16>& buf) {
  using S = VerifyShape<D>;
  const int lane = threadIdx.x, j = lane & 15, g = lane >> 4;
  const uint32_t voff = j * (kGroup / 4) + 8 * g;
  const uint32_t soff = (uint32_t)gi * D * (kGroup / 2) + (uint32_t)half * D * (kGroup / 4);
#pragma unroll
  for (int rt = 0; rt < S::RT; ++rt) {
    const uint32_t o = voff + rt * 16 * (kGroup / 4);
    if constexpr (FMT != kFmtNibble) {  // split layout: channel rows of G/8 bytes per half
      const uint32_t os = j * (kGroup / 8) + 4 * g + rt * 16 * (kGroup / 8);
      const uint32_t ss = (uint32_t)gi * D * (kGroup / 4) + (uint32_t)half * D * (kGroup / 8);
      buf.vu[rt] = split_nibbles(bld4(sm.uv, os, ss), bld4(sm.mv, os, ss));
    } else {
      buf.vu[rt] = bld8(sm.uv, o, soff);
    }
    if constexpr (!UPPER) buf.vl[rt] = bld8(sm.lv, o, soff);
  }
}

template <int D, bool M16>
__device__ __forceinline__ void verify_load_meta(const Streams& sm, int gi, VerifyBuf<D, M16>& buf) {
  // lanes >= D/2 hold no channels and never read km
  buf.km = load_meta<M16>(sm.km, (uint32_t)gi * D);
  buf.vm = load_meta<M16>(sm.vm, (uint32_t)gi * kGroup);
}

// Running state of a verify worker (per lane): softmax max / sum, the value bias sum, and the
// O^T tiles kept in the weight scale of the last group (oinv is its inverse).
template <int D>
struct VerifyAcc {
  float m_run, l_run, beta, oinv;
  f32x4 O[VerifyShape<D>::RT];
};

// One group of a verify worker, in two 64-token halves.  With PF the buffers are refilled with
// group gn as each part of group gi is consumed (a template flag, so that the number of loads in
// flight at every wait is fixed).
template <int D, bool PF, bool UPPER, bool M16, int FMT, class Args, int MQ, bool PAIR>
__device__ __forceinline__ void verify_group(const Args& a, const Streams& sm, VerifyBuf<D, M16>& buf,
                                             int gi, int gn, VerifyLdsQ<MQ, PAIR>& L, VerifyAcc<D>& st) {
  constexpr int COLS = VerifyLdsQ<MQ, PAIR>::kCols;
  using S = VerifyShape<D>;
  const int lane = threadIdx.x;
  // UPPER: every lower nibble is the draft offset
  const uint32_t loff = UPPER ? (uint32_t)a.draft_offset * 0x11111111u : 0u;
  const int j = lane & 15;   // query column
  const int g = lane >> 4;   // k-group
  const int m = a.m;
  const f16x2 c1152 = {(f16)1152.f, (f16)1152.f};
  __syncthreads();  // the previous group's LDS reads are done
  // q' = q s for this lane's channels and every query: fp16 hi/lo into the B-operand slots of
  // the lanes that consume them, and the fp32 bias partials 1024 (q'h + q'l) + q' z (fp16
  // metadata: 1024 (q'h + q'l) - q b, since there a code C stands for s C + b)
  if (lane < D / 2) {
    const float4 km = meta4<M16>(buf.km);
    const float s0 = km.x, z0 = km.y, s1 = km.z, z1 = km.w;
    const int c0 = 2 * lane;
    const int gg = c0 / S::CPL, kk = (c0 % S::CPL) / 8, e0 = c0 % 8;  // e0 even, e0+1 odd
    const int s_even = e0 >> 1, s_odd = 4 + (e0 >> 1);                // slots of e0, e0+1
    f16* bh16 = reinterpret_cast<f16*>(&L.bq[0][kk][COLS * gg]);
    f16* bl16 = PAIR ? bh16 + 8 * 8 : reinterpret_cast<f16*>(&L.bq[PAIR ? 0 : 1][kk][COLS * gg]);
    for (int i = 0; i < m; ++i) {
      {
        const float2 qv = L.qs[i][lane];
        const float qa = qv.x * s0, qb = qv.y * s1;
        f16 ah, al, bhh, bl;
        split_f16(qa, ah, al);
        split_f16(qb, bhh, bl);
        bh16[8 * i + s_even] = ah;
        bl16[8 * i + s_even] = al;
        bh16[8 * i + s_odd] = bhh;
        bl16[8 * i + s_odd] = bl;
        L.bias[i][lane] = 1024.f * (((float)ah + (float)al) + ((float)bhh + (float)bl)) +
                          (M16 ? -(qv.x * z0 + qv.y * z1) : qa * z0 + qb * z1);
      }
    }
  }
  const float4 vm = meta4<M16>(buf.vm);
  L.vm[2 * lane] = make_float2(vm.x, M16 ? fmaf(128.f, vm.x, vm.y) : vm.x * (128.f - vm.y));
  L.vm[2 * lane + 1] = make_float2(vm.z, M16 ? fmaf(128.f, vm.z, vm.w) : vm.z * (128.f - vm.w));
  const float wscale = weight_scale(wave_max_all(fmaxf(vm.x, vm.z)));
  __syncthreads();
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (PF) verify_load_meta<D>(sm, gn, buf);
  f16x8 Bq[S::KK], Bql[S::KK];
#pragma unroll
  for (int kk = 0; kk < S::KK; ++kk) {
    Bq[kk] = __builtin_bit_cast(f16x8, L.bq[0][kk][lane]);
    if constexpr (!PAIR) Bql[kk] = __builtin_bit_cast(f16x8, L.bq[1][kk][lane]);
  }
  // lanes 16g .. 16g+15 of query j, then across the four k-groups (paired form: only the hi
  // columns j < 8 carry it)
  float bias = 0.f;
  {
    const float4* bp = reinterpret_cast<const float4*>(&L.bias[PAIR ? (j & 7) : j][16 * g]);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float4 v = bp[k];
      bias += (v.x + v.y) + (v.z + v.w);
    }
    bias += __shfl_xor(bias, 16);
    bias += __shfl_xor(bias, 32);
    if (PAIR && j >= 8) bias = 0.f;
  }

#pragma unroll
  for (int half = 0; half < 2; ++half) {
    f32x4 St[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < S::KK; ++kk) {
        const f16x8 A = codes_f16(buf.ku[t][kk], UPPER ? loff : buf.kl[t][kk]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, Bq[kk], acc, 0, 0, 0);
        if constexpr (!PAIR) acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, Bql[kk], acc, 0, 0, 0);
      }
      St[t] = acc - bias;
      if constexpr (PAIR) {  // hi products of column j plus lo products of column j ^ 8
#pragma unroll
        for (int i = 0; i < 4; ++i) St[t][i] += dpp<kDppRor8>(St[t][i]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_sched_barrier(0);
    // next key half: the other half of this group, or the first half of the next group
    if (half == 0)
      verify_load_k<D, UPPER, FMT>(sm, gi, 1, buf);
    else if constexpr (PF)
      verify_load_k<D, UPPER, FMT>(sm, gn, 0, buf);
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < 4; ++t)
      mx = fmaxf(mx, fmaxf(fmaxf(St[t][0], St[t][1]), fmaxf(St[t][2], St[t][3])));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(st.m_run, mx);
    const float alpha = fast_exp2(st.m_run - m_new);
    st.m_run = m_new;
    st.l_run *= alpha;
    st.beta *= alpha;
    // O is kept in the weight scale of the current group
    const float oscale = alpha * (wscale * st.oinv);
    st.oinv = 1.f / wscale;
#pragma unroll
    for (int rt = 0; rt < S::RT; ++rt) st.O[rt] *= oscale;
    f16 ph[4][4], pl[4][4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = fast_exp2(St[t][i] - m_new);
        const float2 sw = L.vm[64 * half + 16 * g + 8 * (t >> 1) + 2 * i + (t & 1)];
        st.l_run += p;
        st.beta += p * sw.y;
        split_f16(wscale * (p * sw.x), ph[t][i], pl[t][i]);
        if constexpr (PAIR) ph[t][i] = (j & 8) ? pl[t][i] : ph[t][i];
      }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const f16x8 Bp = {ph[2 * q][0], ph[2 * q][1], ph[2 * q][2], ph[2 * q][3],
                        ph[2 * q + 1][0], ph[2 * q + 1][1], ph[2 * q + 1][2], ph[2 * q + 1][3]};
      const f16x8 Bpl = {pl[2 * q][0], pl[2 * q][1], pl[2 * q][2], pl[2 * q][3],
                         pl[2 * q + 1][0], pl[2 * q + 1][1], pl[2 * q + 1][2], pl[2 * q + 1][3]};
#pragma unroll
      for (int rt = 0; rt < S::RT; ++rt) {
        const uint32_t uw = q == 0 ? buf.vu[rt].x : buf.vu[rt].y;
        const uint32_t lw = UPPER ? loff : (q == 0 ? buf.vl[rt].x : buf.vl[rt].y);
        f16x8 A = codes_f16(uw, lw);
        const f16x2 a0 = f16x2{A[0], A[1]} - c1152, a1 = f16x2{A[2], A[3]} - c1152;
        const f16x2 a2 = f16x2{A[4], A[5]} - c1152, a3 = f16x2{A[6], A[7]} - c1152;
        A = f16x8{a0.x, a0.y, a1.x, a1.y, a2.x, a2.y, a3.x, a3.y};
        st.O[rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, Bp, st.O[rt], 0, 0, 0);
        if constexpr (!PAIR) st.O[rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, Bpl, st.O[rt], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (half == 0)
      verify_load_v<D, UPPER, FMT>(sm, gi, 1, buf);
    else if constexpr (PF)
      verify_load_v<D, UPPER, FMT>(sm, gn, 0, buf);
  }
}

template <int D, bool UPPER, bool M16, int FMT, class Args, int MQ, bool PAIR>
__device__ void verify_quant_item(const Args& a, int b, int h, int item, VerifyLdsQ<MQ, PAIR>& L) {
  constexpr int NBQ = VerifyLdsQ<MQ, PAIR>::kPlanes * 4 * 4 * VerifyLdsQ<MQ, PAIR>::kCols;
  using S = VerifyShape<D>;
  const int lane = threadIdx.x;
  const int j = lane & 15;   // query column
  const int g = lane >> 4;   // k-group
  const int m = a.m;
  const size_t bh = (size_t)b * a.H + h;
  const GroupStride gs = worker_groups(a, b, item);

  // q times qscale of channels 2*lane, 2*lane+1 for every query, and zeroed B operands so the
  // padding query columns j >= m stay zero
  if (lane < D / 2)
    for (int i = 0; i < m; ++i) {
      const uint32_t qq = reinterpret_cast<const uint32_t*>(a.q + qrow(a, b, h, i) * D)[lane];
      L.qs[i][lane] = make_float2(lo_h(qq) * a.qscale, hi_h(qq) * a.qscale);
    }
  for (int x = lane; x < NBQ; x += 64) (&L.bq[0][0][0])[x] = make_uint4(0, 0, 0, 0);
  for (int x = lane; x < MQ * 64; x += 64) (&L.bias[0][0])[x] = 0.f;

  VerifyAcc<D> st;
  st.m_run = -INFINITY;
  st.l_run = 0.f;
  st.beta = 0.f;
  st.oinv = 1.f;
#pragma unroll
  for (int rt = 0; rt < S::RT; ++rt) st.O[rt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const Streams sm = make_streams<M16, FMT>(a, bh, D);
  VerifyBuf<D, M16> buf;
  if (gs.first < gs.ng) {
    verify_load_k<D, UPPER, FMT>(sm, gs.first, 0, buf);
    verify_load_meta<D>(sm, gs.first, buf);
    verify_load_v<D, UPPER, FMT>(sm, gs.first, 0, buf);
    const int total = (gs.ng - gs.first + gs.step - 1) / gs.step;
    int gi = gs.first, done = 0;
    for (; gi + gs.step < gs.ng; gi += gs.step, ++done) {
      pace(total - done, total);
      verify_group<D, true, UPPER, M16, FMT>(a, sm, buf, gi, gi + gs.step, L, st);
    }
    pace(1, total);
    verify_group<D, false, UPPER, M16, FMT>(a, sm, buf, gi, -1, L, st);
  }

  st.l_run += __shfl_xor(st.l_run, 16);
  st.l_run += __shfl_xor(st.l_run, 32);
  st.beta += __shfl_xor(st.beta, 16);
  st.beta += __shfl_xor(st.beta, 32);
  if constexpr (PAIR) {  // O^T column j + 8 holds the lo part of query column j
#pragma unroll
    for (int rt = 0; rt < S::RT; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) st.O[rt][i] += dpp<kDppRor8>(st.O[rt][i]);
  }
  if (j < m) {
    float* rec = record(a, D, b, h, item, j);
    if (g == 0) {
      rec[0] = st.m_run;
      rec[1] = st.l_run;
    }
#pragma unroll
    for (int rt = 0; rt < S::RT; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) rec[kRecPad + 16 * rt + 4 * g + i] = fmaf(st.O[rt][i], st.oinv, st.beta);
  }
}

// ------------------------------------------------------------------------------------------
// Tail work item: up to 64 fp16 tail tokens, m queries, causal (VALU)
// ------------------------------------------------------------------------------------------

struct TailLds {
  uint32_t q[QS_MAX_QUERIES][64];    // fp16 pairs of the m queries, packed: query i at word i*D/2
  float p[kTailChunk][QS_MAX_QUERIES];
};

template <int D, class Args>
__device__ void tail_item(const Args& a, int b, int h, int chunk, int split, TailLds& L) {
  const int lane = threadIdx.x;
  const int m = a.m;
  const int nt = seq_nt(a, b);
  const int ring = 2 * kGroup;
  const size_t bh = (size_t)b * a.H + h;
  const int t0 = chunk * kTailChunk;
  if (Args::kMode == kModeDev && t0 >= nt) {  // device mode plans 2G / 64 chunks: this one is empty
    for (int i = 0; i < m; ++i) {
      float* rec = record(a, D, b, h, split, i);
      if (lane == 0) {
        rec[0] = -INFINITY;
        rec[1] = 0.f;
      }
      for (int c = lane; c < D; c += 64) rec[kRecPad + c] = 0.f;
    }
    return;
  }
  const int t = t0 + lane;                   // logical tail position of this lane's key
  const bool valid = t < nt;
  const int nvalid = min(kTailChunk, nt - t0);
  // head and t0 are multiples of 64, so the chunk's ring slots s0 .. s0 + 63 never wrap
  const int s0 = (seq_head(a, b) + t0) % ring;
  const uint16_t* kchunk = a.tail_k + (bh * ring + s0) * D;
  const uint16_t* vchunk = a.tail_v + (bh * ring + s0) * D;
  if constexpr (Args::kMode == kModeAppend) {
    // fused append: tail positions nt_old .. nt-1 are the tokens this call appends (row i of the
    // append at ak / av + ((b * an_max + i) * H + h) * D).  This item copies the ones in its
    // chunk to their ring slots and waits until the stores are done, then reads the chunk from
    // the ring like any other (no other item reads these slots).
    const int nt_old = nt - a.an[b];
    const int r0 = max(t0, nt_old), r1 = min(t0 + kTailChunk, nt);
    for (int x = lane; x < (r1 - r0) * (D / 8); x += 64) {
      const int r = r0 + x / (D / 8), c = x % (D / 8);
      const size_t src = (((size_t)b * a.an_max + (r - nt_old)) * a.H + h) * D + 8 * c;
      const size_t dst = (bh * ring + s0 + (r - t0)) * D + 8 * c;
      *reinterpret_cast<uint4*>(a.wtail_k + dst) = ld16(a.ak + src);
      *reinterpret_cast<uint4*>(a.wtail_v + dst) = ld16(a.av + src);
    }
    __builtin_amdgcn_s_waitcnt(0);  // every counter drained: the stores have completed
  }

  // The loads of the queries (m * D/2 words, in lane-strided order) and of this lane's key row
  // are issued together before their first use; slots past the nt valid tokens are read (they
  // lie inside the ring) and zeroed.
  constexpr int QW = QS_MAX_QUERIES * (D / 2) / 64;  // query words per lane, at most
  const uint32_t* qsrc = reinterpret_cast<const uint32_t*>(a.q);
  uint32_t qw[QW];
#pragma unroll
  for (int k = 0; k < QW; ++k) {
    const int w = lane + 64 * k;            // word w of the m x D/2 query block
    const int i = w / (D / 2), c = w % (D / 2);
    qw[k] = i < m ? qsrc[qrow(a, b, h, i) * (D / 2) + c] : 0u;
  }
  uint32_t kr[D / 2];
#pragma unroll
  for (int c = 0; c < D / 2; c += 4) {
    const uint4 w = ld16(kchunk + (size_t)lane * D + 2 * c);
    kr[c] = valid ? w.x : 0u;
    kr[c + 1] = valid ? w.y : 0u;
    kr[c + 2] = valid ? w.z : 0u;
    kr[c + 3] = valid ? w.w : 0u;
  }
#pragma unroll
  for (int k = 0; k < QW; ++k) (&L.q[0][0])[lane + 64 * k] = qw[k];
  __syncthreads();

  for (int i = 0; i < m; ++i) {
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < D / 2; ++c) s = dot2(as_h2(kr[c]), as_h2(L.q[0][i * (D / 2) + c]), s);
    s *= a.qscale;
    const bool vis = valid && t <= nt - n_tokens(a) + col_token(a, i);
    if (!vis) s = -INFINITY;
    const float mx = wave_max_from(s, 1);
    const float p = vis ? fast_exp2(s - mx) : 0.f;
    const float sum = wave_sum_from(p, 1);
    if (lane == 0) {
      float* rec = record(a, D, b, h, split, i);
      rec[0] = mx;
      rec[1] = sum;
    }
    L.p[lane][i] = p;
  }
  __syncthreads();

  // o_i[d] = sum_t p_i[t] v_t[d]; lane owns channels lane*CPL ..  The value words of the chunk
  // are loaded in two batches of half a chunk, each batch issued before its first use.
  constexpr int CPL = D / 64;
  constexpr int HB = kTailChunk / 2;
  float acc[QS_MAX_QUERIES][CPL];
#pragma unroll
  for (int i = 0; i < QS_MAX_QUERIES; ++i)
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[i][c] = 0.f;
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    uint32_t vw[HB];
#pragma unroll
    for (int u = 0; u < HB; ++u) {
      const int tt = hb * HB + u;
      uint32_t w;
      if constexpr (CPL == 2)
        w = reinterpret_cast<const uint32_t*>(vchunk + tt * D)[lane];
      else
        w = vchunk[tt * D + lane];
      vw[u] = tt < nvalid ? w : 0u;
    }
#pragma unroll
    for (int i = 0; i < QS_MAX_QUERIES; ++i) {
      if (i < m) {
#pragma unroll
        for (int u = 0; u < HB; ++u) {
          const float p = L.p[hb * HB + u][i];
          if constexpr (CPL == 2) {
            acc[i][0] = fmaf(p, lo_h(vw[u]), acc[i][0]);
            acc[i][1] = fmaf(p, hi_h(vw[u]), acc[i][1]);
          } else {
            acc[i][0] = fmaf(p, (float)__builtin_bit_cast(f16, (uint16_t)vw[u]), acc[i][0]);
          }
        }
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

// Workgroup i of a launch is dispatched to XCD i % kXcds.  The attention kernel renumbers its
// workgroups so that each XCD receives one contiguous range of (head, item) blocks: the XCD then
// streams whole heads, whose planes the address interleave spreads over every HBM channel.  With
// the plain numbering, an XCD's share of a head is every kXcds-th item, and for some grid widths
// those items all read groups with the same low address bits; the call time then varied by more
// than 10% with the item count.
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_contiguous_block(int i, int n) {
  const int x = i % kXcds, k = i / kXcds;
  const int per = n / kXcds, rem = n % kXcds;
  return x * per + (x < rem ? x : rem) + k;  // XCD x holds blocks [start_x, start_x + count_x)
}

template <int NB>
__device__ __forceinline__ int find_seq(const int32_t* base, int B, int idx) {
  int b = 0;
  while (b + 1 < NB && b + 1 < B && base[b + 1] <= idx) ++b;
  return b;
}

// The draft pass runs the VALU item (3 waves per SIMD), except over grouped queries, where both
// passes run the MFMA item: the draft in the paired form (PAIR, up to kPairMaxQueries query
// columns; 11 KB of LDS and 3 waves per SIMD), the verify (and a draft of more columns) in the
// 16-column form (21 KB, 2 waves per SIMD).
template <int D, bool DRAFT, int NB, int MODE, bool M16, int FMT = kFmtNibble, bool PAIR = false>
__global__ __launch_bounds__(64, (DRAFT && (MODE != kModeGqa || PAIR)) ? 3 : 2) void attn_kernel(
    const AttnArgsN<NB, MODE> a) {
  constexpr bool kValu = DRAFT && MODE != kModeGqa;
  using PassLds = typename std::conditional<kValu, DraftLds,
      typename std::conditional<PAIR, VerifyLdsPair, VerifyLds>::type>::type;
  __shared__ union {
    PassLds p;
    TailLds t;
  } lds;
  const int lb = xcd_contiguous_block(blockIdx.y * gridDim.x + blockIdx.x, gridDim.x * gridDim.y);
  const int h = lb / gridDim.x;
  const int x = lb % gridDim.x;
  if (x < a.n_titems_total) {
    const int b = find_seq<NB>(a.titem_base, a.B, x);
    const int chunk = x - a.titem_base[b];
    const int split = (a.qitem_base[b + 1] - a.qitem_base[b]) + chunk;
    tail_item<D>(a, b, h, chunk, split, lds.t);
  } else {
    const int y = x - a.n_titems_total;
    const int b = find_seq<NB>(a.qitem_base, a.B, y);
    const int item = y - a.qitem_base[b];
    if constexpr (kValu)
      draft_quant_item<D, M16, FMT>(a, b, h, item, lds.p);
    else
      verify_quant_item<D, DRAFT, M16, FMT>(a, b, h, item, lds.p);
  }
}

// out[(b, i, h)] = sum_s o_s 2^(m_s - M) / sum_s l_s 2^(m_s - M) over the splits s of (b, h),
// M = max_s m_s.  256 threads in NP phases of D/4 threads: phase p merges the splits p, p + NP,
// .. sixteen at a time (all of a batch's loads issued before its first use; each batch max-first,
// then one log-sum-exp step into the phase's running result), then the phases are merged through
// LDS, max-first as well.
__device__ __forceinline__ void lse_merge(float& m, float& l, float4& o, float m2, float l2,
                                          float4 o2) {
  const float mn = fmaxf(m, m2);
  const float a1 = m == -INFINITY ? 0.f : fast_exp2(m - mn);
  const float a2 = m2 == -INFINITY ? 0.f : fast_exp2(m2 - mn);
  m = mn;
  l = l * a1 + l2 * a2;
  o.x = o.x * a1 + o2.x * a2;
  o.y = o.y * a1 + o2.y * a2;
  o.z = o.z * a1 + o2.z * a2;
  o.w = o.w * a1 + o2.w * a2;
}

// FMT (the upper-plane layout of the attention kernel it follows) only keeps the instantiations
// of the launcher translation units apart.
template <int D, int NB, int MODE, int FMT = kFmtNibble>
__global__ __launch_bounds__(256) void combine_kernel(const AttnArgsN<NB, MODE> a) {
  constexpr int C4 = D / 4;        // float4 chunks of o
  constexpr int NP = 256 / C4;     // split phases
  __shared__ float4 po[NP][C4];
  __shared__ float2 pml[NP];
  // same XCD-contiguous numbering as the attention kernel, so that a head's partials are merged
  // on the XCD that wrote them
  const int lb = xcd_contiguous_block(blockIdx.y * gridDim.x + blockIdx.x, gridDim.x * gridDim.y);
  const int h = lb / gridDim.x;
  const int b = (lb % gridDim.x) / a.m;
  const int i = (lb % gridDim.x) % a.m;
  const int t = threadIdx.x;
  const int c = t % C4, p = t / C4;
  const int ns = (a.qitem_base[b + 1] - a.qitem_base[b]) + (a.titem_base[b + 1] - a.titem_base[b]);
  if constexpr (MODE == kModeDev) {
    if (h == 0 && i == 0 && t == 0) {
      // device mode: the checks the host cannot make, and the commit of the pending operations
      // (every attention item has read the counters by now)
      int32_t bad = 0;
      const int nq = seq_nq(a, b);
      const int nt = apply_pending(a.dev.dstate[kStateInts * b + 1], a.dev.pend, b, &bad);
      if (nq + nt == 0 || nt < a.dev.min_nt) bad |= kDevErrAttend;
      if (bad) atomicOr(a.dev.derr, bad);
      if (a.dev.pend.count) a.dev.wstate[kStateInts * b + 1] = nt;
    }
  }

  float m = -INFINITY, l = 0.f;
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = p; s0 < ns; s0 += NP * 16) {
    float2 ml[16];
    float4 ov[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int s = s0 + NP * u;
      const float* rec = record(a, D, b, h, s < ns ? s : 0, i);
      ml[u] = *reinterpret_cast<const float2*>(rec);
      ov[u] = reinterpret_cast<const float4*>(rec + kRecPad)[c];
      if (s >= ns) {
        ml[u] = make_float2(-INFINITY, 0.f);
        ov[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    // the batch's largest max first, then its weighted sums: independent terms instead of a
    // chain of sixteen rescalings (a record with max -inf weighs 0)
    float bm = ml[0].x;
#pragma unroll
    for (int u = 1; u < 16; ++u) bm = fmaxf(bm, ml[u].x);
    if (bm != -INFINITY) {
      float bl = 0.f;
      float4 bo = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const float w = fast_exp2(ml[u].x - bm);
        bl = fmaf(ml[u].y, w, bl);
        bo.x = fmaf(ov[u].x, w, bo.x);
        bo.y = fmaf(ov[u].y, w, bo.y);
        bo.z = fmaf(ov[u].z, w, bo.z);
        bo.w = fmaf(ov[u].w, w, bo.w);
      }
      lse_merge(m, l, o, bm, bl, bo);
    }
  }
  po[p][c] = o;
  if (c == 0) pml[p] = make_float2(m, l);
  __syncthreads();
  if (t < C4) {
    // the phases, max first as above (mm is finite unless the sequence holds no token, which
    // the host verbs reject and device mode flags in its error word)
    float mm = pml[0].x;
#pragma unroll
    for (int q = 1; q < NP; ++q) mm = fmaxf(mm, pml[q].x);
    float ll = 0.f;
    float4 oo = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int q = 0; q < NP; ++q) {
      const float w = fast_exp2(pml[q].x - mm);
      const float4 v = po[q][t];
      ll = fmaf(pml[q].y, w, ll);
      oo.x = fmaf(v.x, w, oo.x);
      oo.y = fmaf(v.y, w, oo.y);
      oo.z = fmaf(v.z, w, oo.z);
      oo.w = fmaf(v.w, w, oo.w);
    }
    const float inv = 1.f / ll;
    float4* out = reinterpret_cast<float4*>(a.out + qrow(a, b, h, i) * D);
    out[t] = make_float4(oo.x * inv, oo.y * inv, oo.z * inv, oo.w * inv);
  }
}

// ------------------------------------------------------------------------------------------
// Append: n[b] rows of fp16 K/V per sequence into the ring
// ------------------------------------------------------------------------------------------

template <int D, int NB>
__global__ __launch_bounds__(256) void append_kernel(const AppendArgsN<NB> a) {
  constexpr int CH = D / 8;  // 16-byte chunks per row
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  const int row = idx / CH, c = idx % CH;
  const int h = row % a.H;
  const int i = (row / a.H) % a.n_rows;
  const int b = row / (a.H * a.n_rows);
  if (b >= a.B || i >= a.n[b]) return;
  const int ring = 2 * kGroup;
  int start = a.start[b], head = a.head[b];
  if (a.dstate) {  // device mode: an append past the ring writes nothing (flagged at the commit)
    start = apply_pending(a.dstate[kStateInts * b + 1], a.pend, b, nullptr);
    head = a.dstate[kStateInts * b + 2];
    if (start + a.n[b] > ring) return;
  }
  const int slot = (head + start + i) % ring;
  const size_t src = (((size_t)b * a.n_max + a.src0[b] + i) * a.H + h) * D + 8 * c;
  const size_t dst = (((size_t)b * a.H + h) * ring + slot) * D + 8 * c;
  *reinterpret_cast<uint4*>(a.tail_k + dst) = ld16(a.k + src);
  *reinterpret_cast<uint4*>(a.tail_v + dst) = ld16(a.v + src);
}

// ------------------------------------------------------------------------------------------
// Quantizer: one G-token group of (layer, b, h) into both planes and its metadata -- the flush
// (the ring's oldest half) and the prefill (a prompt's whole groups)
// ------------------------------------------------------------------------------------------
//
// Quantizer, in fp32 and in this order (QuantSpec Guide, quantizer listing):
//   s = max((max - min) / 255, 1e-8);  z = rint(-min / s);  c = clamp(rint(x / s) + z, 0, 255)
// keys: one (s, z) per channel over the G tokens; values: one per token over D channels.
// Four-wave workgroups each own a whole (group, head) of keys or of values, so that every load
// reads whole head rows and every store writes whole plane lines.

// (mx - mn) / 255 correctly rounded, as q0 = d y, q = fma(fma(-q0, 255, d), y, q0) with
// y = 1/255 correctly rounded (Markstein's correction step, three instructions instead of an
// IEEE division): for every pair of finite fp16 values the same scale as the division once
// clamped (an unclamped difference only in the sign of a zero difference), checked on the CPU.
__device__ __forceinline__ float quant_scale(float mn, float mx) {
#pragma clang fp contract(off)
  const float d = mx - mn;
  constexpr float y = 1.0f / 255.0f;
  const float q0 = d * y;
  const float s = __builtin_fmaf(__builtin_fmaf(-q0, 255.0f, d), y, q0);
  return s < 1e-8f ? 1e-8f : s;
}
// x / s, correctly rounded, from y = 1 / s (correctly rounded, once per scale) and one
// fma-corrected product: q0 = x y is within an ulp of x / s, the residual x - q0 s is exact in
// an fma, and q0 + r y rounded once is the correctly rounded quotient (Markstein's theorem on
// division by reciprocal and correction; the operands here are finite, with no underflow).
// Three instructions instead of the ~10 of an IEEE division per element; the codes stay
// bit-identical to those of x / s.
__device__ __forceinline__ float div_by(float x, float s, float y) {
  const float q0 = x * y;
  const float r = __builtin_fmaf(-q0, s, x);
  return __builtin_fmaf(r, y, q0);
}
// z = rint(-mn / s) through the codes' division (-mn is an fp16 value), its sign that of -mn as
// the division's is: the corrected quotient of a zero is +0 whatever the zero's sign, and the
// zero-point is stored bit for bit.
__device__ __forceinline__ float zero_point(float mn, float s, float y) {
  return copysignf(rintf(div_by(-mn, s, y)), -mn);
}

// The code (an integer in [0, 255], held as a float) as byte `sel` of acc: v_cvt_pk_u8_f32 converts
// and inserts in one instruction, exactly since the value is already an integer in range.
__device__ __forceinline__ uint32_t put_code(float c, int sel, uint32_t acc) {
  return __builtin_amdgcn_cvt_pk_u8_f32(c, sel, acc);
}
// Packed fp16 minimum / maximum of two words, per half (chains of them become
// v_pk_minimum3_f16 / v_pk_maximum3_f16).
__device__ __forceinline__ uint32_t min_h2(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_minimum(as_h2(a), as_h2(b)));
}
__device__ __forceinline__ uint32_t max_h2(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_maximum(as_h2(a), as_h2(b)));
}
// The code of the fp16 value x in half HI of w, clamped to [0, 255] by one median-of-three (the
// operands are finite): div_by's steps with the first product taken as fma(x, y, +0), which
// v_fma_mix_f32 computes from the half itself (no conversion instruction; the residual's fma
// reads it the same way).  It differs from x y only in the sign of a zero product (x = -0),
// which the corrected quotient does not see: both give +0.
template <int HI>
__device__ __forceinline__ float code_h(uint32_t w, float s, float y, float z) {
#pragma clang fp contract(off)
  const float x = HI ? hi_h(w) : lo_h(w);
  const float q0 = __builtin_fmaf(x, y, 0.0f);
  const float q = __builtin_fmaf(__builtin_fmaf(-q0, s, x), y, q0);
  return __builtin_amdgcn_fmed3f(rintf(q) + z, 0.f, 255.f);
}
__device__ __forceinline__ void load8(const float* p, float* out) {
  const float4 a = reinterpret_cast<const float4*>(p)[0], b = reinterpret_cast<const float4*>(p)[1];
  out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
  out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
}
// Upper and lower nibble words of 8 codes: bytes 0..3 of A hold the codes of entries 0, 2, 4, 6,
// those of B entries 1, 3, 5, 7; byte j of u (of l) then holds the upper (lower) nibble of entry
// 2j in bits 0-3 and that of entry 2j + 1 in bits 4-7 -- each a bit-field insert and a shift.
__device__ __forceinline__ void nibble_planes(uint32_t A, uint32_t B, uint32_t& u, uint32_t& l) {
  constexpr uint32_t m = 0x0F0F0F0Fu;
  u = ((A >> 4) & m) | (B & ~m);
  l = (A & m) | ((B << 4) & ~m);
}

// fp16 metadata of a group (keys: a channel; values: a token) with fp32 scale s and zero-point
// z: s and the offset b = -s z (the fp32 product), each rounded to nearest-even fp16, b clamped
// to the finite range first.  A code C then stands for s C + b.
__device__ __forceinline__ uint32_t meta16_pair(float s, float z) {
#pragma clang fp contract(off)
  const float b = fminf(fmaxf(-(s * z), -65504.f), 65504.f);
  const uint32_t hs = __builtin_bit_cast(uint16_t, (_Float16)s);
  const uint32_t hb = __builtin_bit_cast(uint16_t, (_Float16)b);
  return hs | (hb << 16);
}

constexpr int kTileRow = 128 + 8;  // bytes per token row of a value code tile (8-byte aligned)
// A value row's codes into a token-major tile row: the lane holds words k < HALF / 2 of the row
// (word k: channels 8 (2 (k / 4) + hf) + 2 (k % 4) and + 1), so words 4 q .. 4 q + 3 are the 8
// consecutive channels 8 (2 q + hf) .. + 7, stored as one 8-byte write.
template <int HALF>
__device__ __forceinline__ void store_code_row(const uint32_t* w, float s, float y, float z, int hf,
                                               uint8_t* row) {
#pragma unroll
  for (int q = 0; q < HALF / 8; ++q) {
    uint32_t c[2] = {0, 0};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      c[i >> 1] = put_code(code_h<0>(w[4 * q + i], s, y, z), 2 * (i & 1), c[i >> 1]);
      c[i >> 1] = put_code(code_h<1>(w[4 * q + i], s, y, z), 2 * (i & 1) + 1, c[i >> 1]);
    }
    *reinterpret_cast<uint2*>(row + 8 * (2 * q + hf)) = make_uint2(c[0], c[1]);
  }
}
// One channel's plane words over NT tokens of a token-major tile (col = the channel's byte in
// token row 0): word i covers tokens 8 i .. 8 i + 7.
template <int NT>
__device__ __forceinline__ void tile_column_planes(const uint8_t* col, uint32_t* u, uint32_t* l) {
#pragma unroll
  for (int i = 0; i < NT / 8; ++i) {
    uint32_t A = 0, B = 0;  // tokens 8 i + 2 j (A) and 8 i + 2 j + 1 (B) as byte j
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      A |= (uint32_t)col[(8 * i + 2 * j) * kTileRow] << (8 * j);
      B |= (uint32_t)col[(8 * i + 2 * j + 1) * kTileRow] << (8 * j);
    }
    nibble_planes(A, B, u[i], l[i]);
  }
}

// Per-channel key scales of one block.  The lanes first reduce their rows to packed fp16 partial
// minima / maxima (exact: a minimum of fp16 values is one of them), one partial per wave in mn /
// mx; thread t < NC then takes channel t's (s, 1/s, z) over the NW partials, stores them in s / y
// / z for every lane of the block, and writes the channel's metadata -- once per channel rather
// than once per lane that quantizes it.
template <int NC, int NW>
struct KeyScaleLds {
  uint32_t mn[NW][NC / 2];  // packed fp16 partials: word i = channels 2 i, 2 i + 1
  uint32_t mx[NW][NC / 2];
  float s[NC], y[NC], z[NC];
};

template <int NC, int NW, class Args>
__device__ __forceinline__ void key_scales(const Args& a, KeyScaleLds<NC, NW>& L, size_t pair0) {
  const int t = threadIdx.x;
  if (t < NC) {
    float mn = INFINITY, mx = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      mn = fminf(mn, (float)reinterpret_cast<const f16*>(L.mn[ww])[t]);
      mx = fmaxf(mx, (float)reinterpret_cast<const f16*>(L.mx[ww])[t]);
    }
    const float s = quant_scale(mn, mx);
    const float y = 1.0f / s;
    const float z = zero_point(mn, s, y);
    L.s[t] = s;
    L.y[t] = y;
    L.z[t] = z;
    if (a.meta16)
      *reinterpret_cast<uint32_t*>(a.kmeta + (pair0 + t) * 4) = meta16_pair(s, z);
    else
      *reinterpret_cast<float2*>(a.kmeta + (pair0 + t) * 8) = make_float2(s, z);
  }
}

// Packed minima / maxima of a lane's 8 channels (words wi: channels 2 wi, 2 wi + 1) over its NL
// rows, reduced over the lanes whose lane bits from `first` up differ (same channels, other
// rows), and stored as partial `slot` of channels 8 c .. 8 c + 7 by the lanes with no such bits.
template <int NL, int NC, int NW>
__device__ __forceinline__ void key_partials(const uint4* v, int first, int c, int slot,
                                             KeyScaleLds<NC, NW>& L) {
  uint32_t pmn[4] = {v[0].x, v[0].y, v[0].z, v[0].w}, pmx[4] = {v[0].x, v[0].y, v[0].z, v[0].w};
#pragma unroll
  for (int k = 1; k < NL; ++k) {
    const uint32_t w4[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
#pragma unroll
    for (int wi = 0; wi < 4; ++wi) {
      pmn[wi] = min_h2(pmn[wi], w4[wi]);
      pmx[wi] = max_h2(pmx[wi], w4[wi]);
    }
  }
#pragma unroll
  for (int o = first; o < 64; o <<= 1)
#pragma unroll
    for (int wi = 0; wi < 4; ++wi) {
      pmn[wi] = min_h2(pmn[wi], __shfl_xor(pmn[wi], o));
      pmx[wi] = max_h2(pmx[wi], __shfl_xor(pmx[wi], o));
    }
  if ((threadIdx.x & 63) < first) {
    *reinterpret_cast<uint4*>(&L.mn[slot][4 * c]) = make_uint4(pmn[0], pmn[1], pmn[2], pmn[3]);
    *reinterpret_cast<uint4*>(&L.mx[slot][4 * c]) = make_uint4(pmx[0], pmx[1], pmx[2], pmx[3]);
  }
}

// One key row of a lane: codes of its 8 channels (scales sc / yc / zc) as the row's 4 bytes of
// each plane.  Split-upper layout: lane pair (c even, c odd) shares word c / 2 of the top and
// middle planes; the even lane returns the top word, the odd one the middle word.
__device__ __forceinline__ void key_row(const uint4& v, const float* sc, const float* yc,
                                        const float* zc, bool split, bool odd, uint32_t& hi_word,
                                        uint32_t& lo_word) {
  const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
  uint32_t A = 0, B = 0, u, l;  // codes of the even / odd channels of the lane's 8
#pragma unroll
  for (int wi = 0; wi < 4; ++wi) {
    A = put_code(code_h<0>(w4[wi], sc[2 * wi], yc[2 * wi], zc[2 * wi]), wi, A);
    B = put_code(code_h<1>(w4[wi], sc[2 * wi + 1], yc[2 * wi + 1], zc[2 * wi + 1]), wi, B);
  }
  nibble_planes(A, B, u, l);
  if (split) {
    // nibble e of u is C_U of entry e: entries 0..7 keep C_T in the upper and C_M in the lower
    // two bits of their nibble, entries 8..15 the other way round
    const uint32_t t = odd ? (u >> 2) & 0x33333333u : u & 0xCCCCCCCCu;
    const uint32_t m = odd ? (u << 2) & 0xCCCCCCCCu : u & 0x33333333u;
    const uint32_t other = __shfl_xor(odd ? t : m, 1);  // what the neighbour lacks
    u = (odd ? m : t) | other;
  }
  hi_word = u;
  lo_word = l;
}

// The scale of a value row over its D channels, held by a lane pair (hf = 0, 1) as HALF / 2
// words each: packed minima / maxima over the lane's words, then over the pair.
template <int NW>
__device__ __forceinline__ void row_min_max(const uint32_t* w, float& mn, float& mx) {
  uint32_t pmn = w[0], pmx = w[0];
#pragma unroll
  for (int k = 1; k < NW; ++k) {
    pmn = min_h2(pmn, w[k]);
    pmx = max_h2(pmx, w[k]);
  }
  mn = fminf(lo_h(pmn), hi_h(pmn));
  mx = fmaxf(lo_h(pmx), hi_h(pmx));
  mn = fminf(mn, __shfl_xor(mn, 1));
  mx = fmaxf(mx, __shfl_xor(mx, 1));
}

constexpr int kQuantWaves = 4;
struct GroupValLds {
  uint8_t code[2][kGroup / 2][kTileRow];  // per half group: codes, token-major (padded rows)
};

// Keys of one (group, head), the G fp16 rows at ksrc (token t at ksrc + t * stride), into group
// grp of the quantized tier of (layer, sequence, head) lbh: wave w holds rows 32 w .. 32 w + 31,
// each lane 8 channels (16 bytes) of 32 / RPI of them -- LPR lanes read a row, RPI rows per load instruction.  Each lane
// quantizes its channels of its rows and writes their 4 bytes of each plane row, so a store
// instruction writes RPI whole consecutive rows.
template <int D, class Args>
__device__ void quant_keys(const Args& a, size_t lbh, int grp, const uint16_t* ksrc, size_t stride,
                             KeyScaleLds<D, kQuantWaves>& L) {
  constexpr int G = kGroup, LPR = D / 8, RPI = 64 / LPR, NL = 32 / RPI;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = lane % LPR, r = lane / LPR;  // channels 8 c .. 8 c + 7 of rows 32 w + RPI k + r
  const uint16_t* src = ksrc + 8 * c;
  uint4 v[NL];
#pragma unroll
  for (int k = 0; k < NL; ++k) v[k] = ld16(src + (size_t)(32 * w + RPI * k + r) * stride);
  key_partials<NL>(v, LPR, c, w, L);
  __syncthreads();
  key_scales(a, L, (lbh * a.NG + grp) * D);
  __syncthreads();
  float sc[8], yc[8], zc[8];
  load8(&L.s[8 * c], sc);
  load8(&L.y[8 * c], yc);
  load8(&L.z[8 * c], zc);
  // plane rows: this lane's channels are bytes 4 c .. 4 c + 3 of a row.  Split-upper layout: rows
  // of D/4 bytes in the top and middle planes, word c / 2 of a row holding this lane's 8
  // channels (entries 0..7 if c is even) and its neighbour's
  const size_t row0 = (lbh * a.T + (size_t)grp * G + 32 * w + r) * (D / 2) + 4 * c;
  // the even lane of a pair writes the top plane's word, the odd lane the middle plane's
  uint8_t* const srow = a.uk + lbh * a.T * (D / 2) + ((c & 1) ? (size_t)a.T * (D / 4) : 0) +
                        ((size_t)grp * G + 32 * w + r) * (D / 4) + 4 * (c >> 1);
#pragma unroll
  for (int k = 0; k < NL; ++k) {
    uint32_t u, l;
    key_row(v[k], sc, yc, zc, a.split, c & 1, u, l);
    *reinterpret_cast<uint32_t*>((a.split ? srow + RPI * k * (D / 4) : a.uk + row0 + RPI * k * (D / 2))) = u;
    *reinterpret_cast<uint32_t*>(a.lk + row0 + RPI * k * (D / 2)) = l;
  }
}

// Values of one (group, head), the G fp16 rows at vsrc: wave w quantizes tokens 32 w .. 32 w + 31
// (a lane pair per row: lane hf of the pair takes the row's 16-byte chunks 2 k + hf, so a load
// instruction reads 32 contiguous bytes of every row) into the code tile of its half group; after one barrier wave w
// writes the whole rows of channels (D/2) (w % 2) .. + D/2 - 1 of half w / 2.
template <int D, class Args>
__device__ void quant_values(const Args& a, size_t lbh, int grp, const uint16_t* vsrc, size_t stride,
                               GroupValLds& L) {
  constexpr int G = kGroup, HALF = D / 2;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int half = w >> 1, trow = 32 * (w & 1);  // tokens (G/2) half + trow + tk of the group
  const int tk = lane >> 1, hf = lane & 1;
  const uint16_t* src = vsrc + (size_t)((G / 2) * half + trow + tk) * stride;
  uint32_t wv[HALF / 2];
#pragma unroll
  for (int k = 0; k < HALF / 8; ++k) {
    const uint4 v = ld16(src + 8 * (2 * k + hf));
    wv[4 * k] = v.x; wv[4 * k + 1] = v.y; wv[4 * k + 2] = v.z; wv[4 * k + 3] = v.w;
  }
  float mn, mx;
  row_min_max<HALF / 2>(wv, mn, mx);
  const float s = quant_scale(mn, mx);
  const float y = 1.0f / s;
  const float z = zero_point(mn, s, y);
  if (hf == 0) {
    const size_t pair = lbh * a.T + (size_t)grp * G + (G / 2) * half + trow + tk;
    if (a.meta16)
      *reinterpret_cast<uint32_t*>(a.vmeta + pair * 4) = meta16_pair(s, z);
    else
      *reinterpret_cast<float2*>(a.vmeta + pair * 8) = make_float2(s, z);
  }
  store_code_row<HALF>(wv, s, y, z, hf, &L.code[half][trow + tk][0]);
  __syncthreads();
  // the plane row of channel dch in half `half` holds the half's G/2 tokens, byte j tokens 2j
  // (bits 0-3) and 2j + 1 (bits 4-7)
  const int dch = (D / 2) * (w & 1) + lane;
  if (lane < D / 2) {
    uint32_t u[8], l[8];
    tile_column_planes<G / 2>(&L.code[half][0][dch], u, l);
    const size_t rowb = (((lbh * a.NG + grp) * 2 + half) * D + dch) * (G / 4);
    if (a.split) {
      // a split word covers tokens 16 v .. 16 v + 15: C_T of the first 8 in the upper, of the
      // next 8 in the lower two bits of each nibble, C_M the other way round
      uint32_t t[4], m[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        t[q] = (u[2 * q] & 0xCCCCCCCCu) | ((u[2 * q + 1] >> 2) & 0x33333333u);
        m[q] = (u[2 * q] & 0x33333333u) | ((u[2 * q + 1] << 2) & 0xCCCCCCCCu);
      }
      uint8_t* tv = a.uv + lbh * a.NG * D * (G / 2) + (((size_t)grp * 2 + half) * D + dch) * (G / 8);
      const size_t smid = (size_t)a.NG * D * (G / 4);
      *reinterpret_cast<uint4*>(tv) = make_uint4(t[0], t[1], t[2], t[3]);
      *reinterpret_cast<uint4*>(tv + smid) = make_uint4(m[0], m[1], m[2], m[3]);
    } else {
      *reinterpret_cast<uint4*>(a.uv + rowb) = make_uint4(u[0], u[1], u[2], u[3]);
      *reinterpret_cast<uint4*>(a.uv + rowb + 16) = make_uint4(u[4], u[5], u[6], u[7]);
    }
    *reinterpret_cast<uint4*>(a.lv + rowb) = make_uint4(l[0], l[1], l[2], l[3]);
    *reinterpret_cast<uint4*>(a.lv + rowb + 16) = make_uint4(l[4], l[5], l[6], l[7]);
  }
}

// The rest of a prompt (its tokens after the whole groups) of head h into the ring: rows of D
// fp16, a row's 16-byte chunks over D/8 lanes, 256 / (D/8) rows per pass.
template <int D>
__device__ void prefill_rest(const PrefillArgs& a, int b, int h, const uint16_t* src,
                             uint16_t* ring) {
  constexpr int CH = D / 8, RPP = 64 * kQuantWaves / CH;
  const int c = threadIdx.x % CH;
  for (int i = threadIdx.x / CH; i < a.rest[b]; i += RPP) {
    const int slot = (a.rest_slot[b] + i) % (2 * kGroup);
    const size_t s = (((size_t)b * a.n_max + (size_t)a.groups[b] * kGroup + i) * a.H + h) * D + 8 * c;
    const size_t d = (((size_t)b * a.H + h) * (2 * kGroup) + slot) * D + 8 * c;
    *reinterpret_cast<uint4*>(ring + d) = ld16(src + s);
  }
}

// Prefill: whole groups of a prompt quantized straight from the caller's k / v [B][n_max][H][D]
// (a head's G rows of 2 D bytes lie H * 2 D bytes apart), and the rest of the prompt into the
// ring by the workgroups of row rest_row.
// grid: x = 2 head + kind (0 keys, 1 values), y = prompt group, z = sequence; 256 threads.  Group
// g of sequence b's prompt (its tokens g G .. g G + G - 1) goes to quantized group group0[b] + g.
template <int D>
__global__ __launch_bounds__(64 * kQuantWaves) __attribute__((amdgpu_waves_per_eu(4))) void prefill_kernel(const PrefillArgs a) {
  // 32 KB per workgroup, so that at most five share a compute unit: more in flight only adds
  // contention to the mixed read / write stream (measured at 128k: 608 us with five per unit,
  // 613 us with four, 617 us with seven)
  __shared__ union {
    KeyScaleLds<D, kQuantWaves> k;
    GroupValLds v;
    uint8_t occupancy[32 * 1024];
  } lds;
  const int n = gridDim.x * gridDim.y * gridDim.z;
  const int lb = xcd_contiguous_block((blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x, n);
  const int bx = lb % gridDim.x, g = (lb / gridDim.x) % gridDim.y, b = lb / (gridDim.x * gridDim.y);
  const int h = bx >> 1;
  if (g == a.rest_row) {  // no barriers on this path
    if ((bx & 1) == 0)
      prefill_rest<D>(a, b, h, a.k, a.tail_k);
    else
      prefill_rest<D>(a, b, h, a.v, a.tail_v);
    return;
  }
  if (g >= a.groups[b]) return;  // the whole workgroup, before its barriers
  const size_t lbh = ((size_t)a.layer * a.B + b) * a.H + h;
  const size_t stride = (size_t)a.H * D;
  const size_t src0 = (((size_t)b * a.n_max + (size_t)g * kGroup) * a.H + h) * D;
  if ((bx & 1) == 0)
    quant_keys<D>(a, lbh, a.group0[b] + g, a.k + src0, stride, lds.k);
  else
    quant_values<D>(a, lbh, a.group0[b] + g, a.v + src0, stride, lds.v);
}


// Flush: the ring's oldest half (rows of D fp16, contiguous) of each selected (layer, sequence,
// head) into its next quantized group.
// grid: x = 2 head + kind (0 keys, 1 values), y = selected sequence, z = layer - layer0; 256
// threads.  A whole launch's halves fit in about one resident round of workgroups.
template <int D>
__global__ __launch_bounds__(64 * kQuantWaves) void flush_kernel(const FlushArgs a) {
  __shared__ union {
    KeyScaleLds<D, kQuantWaves> k;
    GroupValLds v;
  } lds;
  const int n = gridDim.x * gridDim.y * gridDim.z;
  const int lb = xcd_contiguous_block((blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x, n);
  const int bx = lb % gridDim.x, sel = (lb / gridDim.x) % gridDim.y, bz = lb / (gridDim.x * gridDim.y);
  const int h = bx >> 1;
  const int layer = a.layer0 + bz;
  const size_t lbh = ((size_t)layer * a.B + a.b[sel]) * a.H + h;
  int group = a.group[sel], head = a.head[sel];
  if (a.dstate) {  // device mode: this sequence flushes only if selected and within capacity
    const int32_t* st = a.dstate + ((size_t)layer * a.B + a.b[sel]) * kStateInts;
    const int nq = st[0], nt = apply_pending(st[1], a.pend, a.b[sel], nullptr);
    if (nt < a.thr || nq + kGroup > a.T) return;  // the whole workgroup, before its barriers
    group = nq / kGroup;
    head = st[2];
  }
  const size_t ring0 = (lbh * (2 * kGroup) + head) * D;  // oldest ring half, token-major
  if ((bx & 1) == 0)
    quant_keys<D>(a, lbh, group, a.tail_k + ring0, D, lds.k);
  else
    quant_values<D>(a, lbh, group, a.tail_v + ring0, D, lds.v);
}

// ------------------------------------------------------------------------------------------
// Launchers (called by the C ABI in qs_api.cpp)
// ------------------------------------------------------------------------------------------

// The first NB entries of the per-sequence arrays of a full-size argument block (the host fills
// the full-size block; the launch passes only the bucket the batch needs).
template <int NB>
AttnArgsN<NB> narrow(const AttnArgs& f) {
  AttnArgsN<NB> a;
  static_cast<AttnHeader&>(a) = f;
  for (int b = 0; b < NB; ++b) {
    a.nq[b] = f.nq[b];
    a.nt[b] = f.nt[b];
    a.head[b] = f.head[b];
  }
  for (int b = 0; b <= NB; ++b) {
    a.qitem_base[b] = f.qitem_base[b];
    a.titem_base[b] = f.titem_base[b];
  }
  return a;
}

template <int NB>
AttnArgsN<NB, kModeDev> narrow(const AttnDevArgs& f) {
  AttnArgsN<NB, kModeDev> a;
  static_cast<AttnArgsN<NB>&>(a) = narrow<NB>(static_cast<const AttnArgs&>(f));
  a.dev = f.dev;
  return a;
}

template <int NB>
AttnArgsN<NB, kModeAppend> narrow(const AttnAppArgs& f) {
  AttnArgsN<NB, kModeAppend> a;
  static_cast<AttnArgsN<NB>&>(a) = narrow<NB>(static_cast<const AttnArgs&>(f));
  a.ak = f.ak;
  a.av = f.av;
  a.wtail_k = f.wtail_k;
  a.wtail_v = f.wtail_v;
  a.an_max = f.an_max;
  for (int b = 0; b < NB; ++b) a.an[b] = f.an[b];
  return a;
}

template <int NB>
AttnArgsN<NB, kModeGqa> narrow(const AttnGqaArgs& f) {
  AttnArgsN<NB, kModeGqa> a;
  static_cast<AttnArgsN<NB>&>(a) = narrow<NB>(static_cast<const AttnArgs&>(f));
  a.gq = f.gq;
  a.mt = f.mt;
  a.hq = f.hq;
  return a;
}

template <int NB>
AppendArgsN<NB> narrow(const AppendArgs& f) {
  AppendArgsN<NB> a;
  static_cast<AppendHeader&>(a) = f;
  for (int b = 0; b < NB; ++b) {
    a.n[b] = f.n[b];
    a.start[b] = f.start[b];
    a.head[b] = f.head[b];
    a.src0[b] = f.src0[b];
  }
  return a;
}

template <int D, bool DRAFT, int MODE, bool M16, int FMT = kFmtNibble, bool PAIR = false>
const void* attn_fn(int bucket) {
  switch (bucket) {
    case 1: return (const void*)attn_kernel<D, DRAFT, 1, MODE, M16, FMT, PAIR>;
    case 8: return (const void*)attn_kernel<D, DRAFT, 8, MODE, M16, FMT, PAIR>;
    default: return (const void*)attn_kernel<D, DRAFT, QS_MAX_BATCH, MODE, M16, FMT, PAIR>;
  }
}

template <int MODE, bool M16, int FMT = kFmtNibble>
const void* attn_fn_dm(int D, bool draft, int bucket) {
  if constexpr (FMT == kFmtSplit2)  // the 2-bit layout serves only the draft
    return D == 128 ? attn_fn<128, true, MODE, M16, FMT>(bucket) : attn_fn<64, true, MODE, M16, FMT>(bucket);
  else
    return D == 128 ? (draft ? attn_fn<128, true, MODE, M16, FMT>(bucket) : attn_fn<128, false, MODE, M16, FMT>(bucket))
                    : (draft ? attn_fn<64, true, MODE, M16, FMT>(bucket) : attn_fn<64, false, MODE, M16, FMT>(bucket));
}

// The grouped-query draft in the paired form (m <= kPairMaxQueries query columns).
template <bool M16>
const void* attn_fn_gqa_pair(int D, int bucket) {
  return D == 128 ? attn_fn<128, true, kModeGqa, M16, kFmtNibble, true>(bucket)
                  : attn_fn<64, true, kModeGqa, M16, kFmtNibble, true>(bucket);
}

template <int D, bool DRAFT, int NB, int MODE, int FMT, class Full>
hipError_t launch_attention_n(const Full& f, hipStream_t st) {
  const AttnArgsN<NB, MODE> a = narrow<NB>(f);
  const dim3 grid(a.n_titems_total + a.n_qitems_total, a.H);
  constexpr bool kMayPair = MODE == kModeGqa && DRAFT && FMT == kFmtNibble;
  if constexpr (FMT != kFmtNibble)  // the split layout is built with fp32 metadata only
    hipLaunchKernelGGL((attn_kernel<D, DRAFT, NB, MODE, false, FMT>), grid, dim3(64), 0, st, a);
  else if (kMayPair && gqa_paired(DRAFT, a.m) && a.meta16)
    hipLaunchKernelGGL((attn_kernel<D, DRAFT, NB, MODE, true, FMT, kMayPair>), grid, dim3(64), 0, st, a);
  else if (kMayPair && gqa_paired(DRAFT, a.m))
    hipLaunchKernelGGL((attn_kernel<D, DRAFT, NB, MODE, false, FMT, kMayPair>), grid, dim3(64), 0, st, a);
  else if (a.meta16)
    hipLaunchKernelGGL((attn_kernel<D, DRAFT, NB, MODE, true>), grid, dim3(64), 0, st, a);
  else
    hipLaunchKernelGGL((attn_kernel<D, DRAFT, NB, MODE, false>), grid, dim3(64), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 cgrid(a.B * a.m, a.H);
  hipLaunchKernelGGL((combine_kernel<D, NB, MODE, FMT>), cgrid, dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int D, bool DRAFT, int MODE, int FMT, class Full>
hipError_t launch_attention_d(const Full& a, hipStream_t st) {
  switch (batch_bucket(a.B)) {
    case 1: return launch_attention_n<D, DRAFT, 1, MODE, FMT>(a, st);
    case 8: return launch_attention_n<D, DRAFT, 8, MODE, FMT>(a, st);
    default: return launch_attention_n<D, DRAFT, QS_MAX_BATCH, MODE, FMT>(a, st);
  }
}

template <int MODE, int FMT = kFmtNibble, class Full>
hipError_t launch_attention_m(const Full& a, int D, bool draft, hipStream_t st) {
  if constexpr (FMT == kFmtSplit2) {
    if (!draft) return hipErrorInvalidValue;
    return D == 128 ? launch_attention_d<128, true, MODE, FMT>(a, st) : launch_attention_d<64, true, MODE, FMT>(a, st);
  } else {
    if (D == 128)
      return draft ? launch_attention_d<128, true, MODE, FMT>(a, st) : launch_attention_d<128, false, MODE, FMT>(a, st);
    return draft ? launch_attention_d<64, true, MODE, FMT>(a, st) : launch_attention_d<64, false, MODE, FMT>(a, st);
  }
}

}  // namespace qs
