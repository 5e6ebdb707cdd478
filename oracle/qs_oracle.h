/*
 * qs_oracle.h -- CPU oracle of the hierarchical INT8 KV cache.
 *
 * TEST INFRASTRUCTURE.  This is the plain, slow, obviously-correct reference that the GPU
 * library is checked against.  Only the tests, the smoke check and the CPU-baseline leg of the
 * benchmark may load it; the library never does.  It shares no code with the GPU library.
 *
 * Every function follows the pages' definitions step by step:
 *  - quantizer: asymmetric per-group min/max quantization to 8 bits, computed in fp32
 *    ("Hierarchical Quantizer with Bit-Packing" listing of the QuantSpec Guide);
 *  - split: C_U = C8 >> 4, C_L = C8 & 15, so C8 = 16*C_U + C_L (Pith review of arXiv:2502.10424,
 *    "What carries the argument"; Fig. 3);
 *  - key groups are channel-wise over G tokens, value groups token-wise over the head's
 *    channels (Pith review, Fig. 7 and reference [128]);
 *  - draft dequantization ((16*C_U + off) - z) * s, verify dequantization (C8 - z) * s, both in
 *    fp64 (QuantSpec Guide, unpack_for_draft / unpack_for_target);
 *  - attention: one fp64 softmax over the concatenation of the dequantized quantized tier and
 *    the fp16 tail (the plain definition; the split-softmax merge of the GPU path reaches it
 *    exactly in real arithmetic -- Pith review, reference [128], Flash Decoding);
 *  - tail ring of 2G fp16 slots with append / rollback / flush bookkeeping (QuantSpec Guide,
 *    "3. Double Full-Precision Cache Buffer (CF1 and CF2)"; Pith review, "Core claim").
 *
 * Status codes are the integers 0 (ok), 1 (invalid argument), 2 (capacity), 3 (state).
 */
#ifndef QS_ORACLE_H
#define QS_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* IEEE binary16 bit pattern -> float (exact). */
float orc_half_to_float(uint16_t h);

/* Quantizes one group of n values x[i * stride] (fp16 bit patterns) to codes c[i * cstride];
 * writes the fp32 scale and zero-point. */
void orc_quantize_group(const uint16_t* x, int n, int stride, float* s, float* z, uint8_t* c,
                        int cstride);

/* Dequantizations, in fp64. */
double orc_dequant_full(uint8_t c8, float s, float z);
double orc_dequant_upper(uint8_t cu, float s, float z, int off);
/* Top-k-bit draft dequantization (k in 1..8) of an 8-bit code: the top k bits, the dropped
 * 8 - k bits replaced by off/16 of their range; k = 4 equals orc_dequant_upper(c8 >> 4), k = 8
 * orc_dequant_full.  The fp16-metadata form takes (s, b). */
double orc_dequant_topk(uint8_t c8, float s, float z, int k, int off);
double orc_dequant16_topk(uint8_t c8, float s, float b, int k, int off);

/* fp32 -> binary16 bits, round to nearest even (overflow to infinity). */
uint16_t orc_float_to_half(float x);
/* fp16 metadata of a group with fp32 scale s and zero-point z: the fp16 values (as floats) of
 * s and of the offset b = -(s z) clamped to +-65504. */
void orc_meta16(float s, float z, float* s16, float* b16);
/* Dequantizations with fp16 metadata (s, b), in fp64: s C8 + b and s (16 C_U + off) + b. */
double orc_dequant16_full(uint8_t c8, float s, float b);
double orc_dequant16_upper(uint8_t cu, float s, float b, int off);

typedef struct orc_cache orc_cache;

/* L layers, B sequences, H heads, head_dim D, group G, quantized capacity T (multiple of G),
 * gamma_max, draft offset off, metadata format (0: fp32 (s, z); 1: fp16 (s, b)).  Returns NULL
 * on invalid arguments or allocation failure. */
orc_cache* orc_create(int L, int B, int H, int D, int G, int T, int gamma_max, int off,
                      int meta16);
void orc_destroy(orc_cache* c);

/* k, v: fp16 bits [B][n_max][H][D]; n: [B] or NULL (= n_max). */
int orc_append(orc_cache* c, int layer, const uint16_t* k, const uint16_t* v, int n_max,
               const int* n);
/* Prompt of n[b] tokens per sequence (k, v as for append): whole groups quantized through the
 * buffer, the rest left in it; needs an empty buffer for every sequence with n[b] > 0. */
int orc_prefill(orc_cache* c, int layer, const uint16_t* k, const uint16_t* v, int n_max,
                const int* n);
/* Speculative accept / correct: t fp32 [B][gamma+1][V], d [B][gamma][V], tokens [B][gamma],
 * u [B][gamma+1]; n_acc, next [B]; margin [B] or NULL. */
int orc_spec_accept(const float* t, const float* d, const int* tokens, const float* u, int B,
                    int gamma, int V, int* n_acc, int* next, double* margin);
/* layer -1 = every layer; n_drop: [B] or NULL. */
int orc_rollback(orc_cache* c, int layer, const int* n_drop);
/* layer -1 = every layer; flushed: [B] or NULL. */
int orc_flush(orc_cache* c, int layer, int min_tail, int* flushed);

/* q: fp16 bits [B][H][D]; out [B][H][D]. */
int orc_attend_draft(const orc_cache* c, int layer, const uint16_t* q, double sm_scale,
                     float* out);
/* The draft pass on the top `bits` (1..8) bits of every code; bits = 4 is orc_attend_draft. */
int orc_attend_draft_bits(const orc_cache* c, int layer, const uint16_t* q, int bits,
                          double sm_scale, float* out);
/* q: fp16 bits [B][m][H][D]; out [B][m][H][D]. */
int orc_attend_verify(const orc_cache* c, int layer, const uint16_t* q, int m, double sm_scale,
                      float* out);

int orc_get_state(const orc_cache* c, int layer, int* nq, int* nt, int* head);

/* Logical read-back for one (layer, b, h):
 *   codes  [T][D]   8-bit codes of the quantized tokens (rows >= nq are zero)
 *   kmeta  [T/G][D][2] key (s, z);  vmeta [T][2] value (s, z)  (fp16 format: (s, b)). */
int orc_read_codes(const orc_cache* c, int layer, int b, int h, int which_v, uint8_t* codes);
/* Test support: every stored code of `layer` gets lower nibble `value` (0..15). */
int orc_set_lower_nibbles(orc_cache* c, int layer, int value);
/* Test support: the low nbits (1..7) bits of every stored code of the layer set to value. */
int orc_set_low_bits(orc_cache* c, int layer, int nbits, int value);
/* The split-upper layout's planes of one layer: the top two bits and the middle two bits of
 * every code, as 2-bit planes (key [B][H][T][D/4], value [B][H][T/G][2][D][G/8]); the word
 * arrangement is documented at the definition.  The lower planes, metadata and tail are those
 * of orc_export_layer. */
int orc_export_upper_split(const orc_cache* c, int layer, uint8_t* tk, uint8_t* mk, uint8_t* tv,
                           uint8_t* mv);
int orc_read_meta(const orc_cache* c, int layer, int b, int h, float* kmeta, float* vmeta);

/* Packs one layer into the arena layout of the library (per-layer slices of each section):
 *   uk, lk [B][H][T][D/2]; uv, lv [B][H][T/G][2][D][G/4]; kmeta [B][H][T/G][D][2];
 *   vmeta [B][H][T][2]; tail_k, tail_v [B][H][2G][D] (fp16 bits, the ring slots).
 * Quantized rows >= nq and ring slots never written are zero. */
int orc_export_layer(const orc_cache* c, int layer, uint8_t* uk, uint8_t* lk, uint8_t* uv,
                     uint8_t* lv, float* kmeta, float* vmeta, uint16_t* tail_k,
                     uint16_t* tail_v);

#ifdef __cplusplus
}
#endif

#endif
