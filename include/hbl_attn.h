/*
 * hbl_attn.h -- C ABI of BitNet v2's low-bit attention states for AMD MI355X
 * (gfx950): per-head absmax quantisation of post-RoPE Q/K/V to unsigned
 * integers, a KV cache held in those codes, and one decode step of attention
 * read straight from the packed cache.
 *
 * Source: 新智元 article "微软再放LLM量化大招", section 实验效果 (the QKV
 * states are quantised after RoPE, each head mapped to unsigned integers by
 * absmax with no calibration data; tables 2 and 3 vary the widths), and the
 * 量子位 article on BitNet v2 (a 3-bit KV cache matches the full-precision one).
 *
 * Quantiser, per head (one token's d values v of one head), b bits:
 *     Qb = 2^(b-1) - 1,  Z = 2^(b-1),  G = max(max_e |v_e|, 1e-5 as fp32),
 *     n_e = round_half_even(v_e * Qb / G),  u_e = n_e + Z  (1 <= u_e <= 2^b - 1),
 *     scale = G / Qb (fp32),  value of a code = (u_e - Z) * scale.
 * The decision of every code is exact (no dependence on the rounding of
 * Qb / G): the HIP path gives the same codes as exact arithmetic on the bf16
 * inputs, and scale is the correctly rounded fp32 quotient.
 *
 * Decode attention, for sequence b and query head h (KV head h / (Hq / Hkv)):
 *     q^ = dequantised codes of q (q_bits),   k^_t, v^_t from the cache,
 *     l_t = q^ . k^_t / sqrt(d),  p = softmax(l over t < len_b),
 *     out = sum_t p_t v^_t;   len_b == 0 gives out = 0.
 * The HIP path computes the key dot products exactly in integers and the
 * rest in fp32.
 *
 * Packed code layout (b in {2, 3, 4, 8}): a row of d codes is d/32 groups of
 * 32 consecutive codes; a group is b little-endian 32-bit words w[0..b-1]
 * (4*b bytes), so a row takes d*b/8 bytes.  Code c = 4*q + i of a group
 * (q = 0..7, i = 0..3) lies in byte i of a word as follows:
 *     b = 8: word q, bits 8i..8i+7.
 *     b = 4: word q/2, bits 8i + 4*(q%2) .. +3.
 *     b = 2: word q/4, bits 8i + 2*(q%4) .. +1.
 *     b = 3: q < 6: word q/2, bits 8i + 3*(q%2) .. +2;
 *            q = 6: bits 0-1 at word 0 bits 8i+6..8i+7, bit 2 at word 2 bit 8i+6;
 *            q = 7: bits 0-1 at word 1 bits 8i+6..8i+7, bit 2 at word 2 bit 8i+7.
 * KV cache: codes uint8 [B][Hkv][Tmax][d*b/8], scales fp32 [B][Hkv][Tmax]
 * (row (b*Hkv + h)*Tmax + t is token t of head h of sequence b).
 *
 * Conventions are those of hbl.h: device pointers owned by the caller, 16-byte
 * aligned; asynchronous on `stream`; arguments validated before any launch
 * (nothing is launched on error); gfx950 only.
 * Supported: d in {64, 128, 256}; cache widths b in {2, 3, 4, 8}; query widths
 * q_bits in 2..8; counts (R, B, Tn, Hq, Hkv, Tmax) below 2^31, at most 2^34
 * cache rows (B * Hkv * Tmax), below 2^31 bytes of codes per head
 * (Tmax * d * b / 8) and 2^31 partial records (B * Hq * chunks).
 * Lengths and positions live in device memory, so the host cannot check them:
 * the kernels clamp lengths to [0, Tmax] and skip cache rows whose position
 * falls outside [0, Tmax).  Non-finite inputs give unspecified (but in-bounds)
 * results.
 */
#ifndef HBL_ATTN_H
#define HBL_ATTN_H

#include "hbl.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Quantise R rows (token-heads) of d bf16 values: codes uint8 [R][d*bits/8]
 * in the packed layout, scale fp32 [R].  R == 0 launches nothing. */
hbl_status hbl_quantize_heads(const void *x, int64_t R, int64_t d, int bits,
                              uint8_t *codes, float *scale, hipStream_t stream);

/* Codes -> values (u - Z) * scale, y [R][d] in y_dtype (fp32 or bf16, rounded
 * to nearest even). */
hbl_status hbl_dequantize_heads(const uint8_t *codes, const float *scale, int64_t R, int64_t d,
                                int bits, void *y, hbl_dtype y_dtype, hipStream_t stream);

/* Append Tn new tokens per sequence to a KV cache: k, v bf16 [B][Tn][Hkv][d]
 * (post-RoPE keys and values, as produced by the projections); token t of
 * sequence b goes to cache position pos[b] + t (pos: device int32 [B], or
 * NULL for position 0).  Writes the codes and scales of both tensors. */
hbl_status hbl_kv_cache_append(const void *k, const void *v, int64_t B, int64_t Tn, int64_t Hkv,
                               int64_t d, int bits, const int32_t *pos, int64_t Tmax,
                               uint8_t *k_codes, float *k_scale, uint8_t *v_codes, float *v_scale,
                               hipStream_t stream);

/* Bytes of workspace hbl_attention_decode needs (partial results per chunk
 * of cached tokens). */
size_t hbl_attention_workspace_bytes(int64_t B, int64_t Hq, int64_t d, int64_t Tmax);

/* One decode step: q bf16 [B][Hq][d] (post-RoPE, quantised inside with
 * q_bits), cache as above with kv_bits, lens device int32 [B], out [B][Hq][d]
 * in out_dtype.  Hq must be a multiple of Hkv. */
hbl_status hbl_attention_decode(const void *q, int q_bits, const uint8_t *k_codes,
                                const float *k_scale, const uint8_t *v_codes, const float *v_scale,
                                int kv_bits, const int32_t *lens, int64_t B, int64_t Hq, int64_t Hkv,
                                int64_t d, int64_t Tmax, void *out, hbl_dtype out_dtype,
                                void *workspace, size_t ws_bytes, hipStream_t stream);

/* Causal prefill attention: q bf16 [B][Tn][Hq][d] holds Tn new tokens per
 * sequence (post-RoPE, quantised inside with q_bits), already appended to the
 * cache at positions start[b] .. start[b] + Tn - 1 (start: device int32 [B]);
 * token i attends to cached tokens 0 .. start[b] + i.  out [B][Tn][Hq][d] in
 * out_dtype.  Scores are exact integer dot products on the int8 matrix
 * instruction; the probabilities times the value scales are rounded to bf16
 * for the value product (bf16 matrix instruction, fp32 accumulation).
 * d in {64, 128, 256}.  start[b] is clamped to [0, Tmax] and a query whose
 * position is Tmax or more sees the whole cache (Tmax keys); Tmax + Tn must
 * stay below 2^31 - 512 (HBL_ERR_SHAPE).  No workspace. */
hbl_status hbl_attention_prefill(const void *q, int q_bits, const uint8_t *k_codes, const float *k_scale,
                                 const uint8_t *v_codes, const float *v_scale, int kv_bits,
                                 const int32_t *start, int64_t B, int64_t Tn, int64_t Hq, int64_t Hkv,
                                 int64_t d, int64_t Tmax, void *out, hbl_dtype out_dtype, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* HBL_ATTN_H */
