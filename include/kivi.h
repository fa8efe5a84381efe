/*
 * kivi.h -- C ABI of libkivi: KIVI KV-cache quantization and decode attention
 * over the packed cache, hand-written for AMD CDNA4 (gfx950).
 *
 * What is computed (pages cited by title and section):
 *  - "KIVI - 2-bit KV cache quantisation" (LLM systems cookbook notebook),
 *    "Asymmetric 2-bit quantiser" and "K (per-channel) and V (per-token)
 *    quantisation": per group, zero = min, scale = (max - min) / (2^b - 1)
 *    (scale 1 for a constant group), code = round((x - zero) / scale).
 *  - "KIVI" (VeloxQuant-MLX docs), "How it works": keys are grouped along the
 *    token axis (one group = G tokens of one channel), values along the
 *    channel axis (one group = G channels of one token); the newest R tokens
 *    stay in full precision and older tokens are quantized only in whole
 *    multiples of G, so one-shot prefill and token-by-token decode give the
 *    same cache bit for bit.
 *  - "[Paper review] KIVI ... (ICML'24)", 1.3 (decoding: append the new K/V,
 *    then A = softmax(q K^T), o = A V) and 3.2 system-level implementation
 *    (dequantization fused into the matrix products).
 *
 * Conventions for every entry point:
 *  - Pointers named "device" are HIP device addresses; the library never
 *    allocates, frees or synchronizes; all work is enqueued on the caller's
 *    stream in call order.  Host handles are not thread-safe.
 *  - Arguments are validated before anything is enqueued: a call that fails
 *    validation has had no effect.  KIVI_ERR_HIP means the runtime refused a
 *    kernel launch: launches the call enqueued before it stay enqueued, but
 *    the handle's n and quantized prefixes, the ring and every byte a later
 *    call reads are as they were before the call (the earlier launches only
 *    write packed blocks outside the quantized prefixes), so the call may be
 *    retried.  The one exception is kivi_append_decode when the append part
 *    needs launches of its own (see there).  Asynchronous kernel faults
 *    surface at the caller's next synchronization.
 *  - Inputs must be finite (NaN / Inf are a precondition violation and are
 *    not checked).
 */
#ifndef KIVI_H
#define KIVI_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KIVI_OK = 0,
    KIVI_ERR_INVALID_ARG = 1,      /* bad config, null pointer, bad flag    */
    KIVI_ERR_UNSUPPORTED = 2,      /* valid KIVI, but not a shape built here */
    KIVI_ERR_CAPACITY = 3,         /* n + n_new > max_tokens                 */
    KIVI_ERR_BUFFER_TOO_SMALL = 4, /* device buffer or workspace too small  */
    KIVI_ERR_STATE = 5,            /* decode on an empty / unflushed cache   */
    KIVI_ERR_HIP = 6               /* a kernel launch failed                 */
} kivi_status;

typedef enum { KIVI_F16 = 0, KIVI_F32 = 1 } kivi_dtype;

/* Flush policy: which tokens of an n-token stream are quantized.
   KIVI_FLUSH_WINDOW: keys and values alike up to Q(n) = G * floor(max(0,
   n - R) / G) ("KIVI" VeloxQuant-MLX docs, "How it works" items 3-4: the
   newest R tokens stay full precision, aged tokens move in whole groups).
   KIVI_FLUSH_PAPER (needs R > 0): keys up to Q_K(n) = n - (n mod R), values
   up to Q_V(n) = max(0, n - R) ("[Paper review] KIVI ...", 3.2.2 and the
   prefill / decoding phases of Algorithm 1 in 3.2.3: the key residual is
   quantized R tokens at once when it fills up, the oldest value of the
   residual one token per step).  In the 32-token block holding Q_V the value codes
   and side data of tokens >= Q_V are 0.
   KIVI_FLUSH_SEGMENT (KCVT, the GEAR review's "KCVT" and "streaming buffer
   strategy" sections; needs R > 0 a multiple of 32, G = head_dim, no
   key_outliers): new tokens wait in the full-precision buffer of R tokens
   and keys and values are quantized up to Q(n) = n - (n mod R); each append
   or flush that moves Q quantizes its tokens [Q_old, Q_new) as one segment,
   with one zero / scale per key channel over the whole segment (stored in
   each of its blocks) and one per token over all D value channels. */
typedef enum { KIVI_FLUSH_WINDOW = 0, KIVI_FLUSH_PAPER = 1, KIVI_FLUSH_SEGMENT = 2 } kivi_flush_policy;

/* kivi_append flags. */
enum {
    /* Copy the new rows into the ring only and leave the quantization of
       newly aged groups to a later kivi_flush (or to the next append without
       this flag).  All unquantized tokens must then fit the ring:
       n - G * floor(q_v / G) <= R + G (q_v: quantized value tokens, = q
       under the window policy), else KIVI_ERR_CAPACITY. */
    KIVI_DEFER_FLUSH = 1u
};

typedef struct {
    int32_t batch;        /* B  >= 1                                          */
    int32_t n_kv_heads;   /* H  >= 1                                          */
    int32_t n_q_heads;    /* Hq: a multiple of H; Hq / H in {1, 2, 4}         */
    int32_t head_dim;     /* D: 128                                           */
    int32_t bits;         /* b: 2, 4 or 8                                     */
    int32_t group;        /* G: 32, 64 or 128 (key groups of G tokens, value  */
                          /* groups of G channels)                            */
    int32_t residual;     /* R >= 0, a multiple of G (segment policy: R > 0,  */
                          /* a multiple of 32)                                */
    int32_t kv_dtype;     /* kivi_dtype of the K/V rows handed to append      */
    int32_t policy;       /* kivi_flush_policy                                */
    int32_t key_outliers; /* 0..3: per 32-token key group, this many channels  */
                          /* (the largest max |K|) kept in fp16; 2 is the    */
                          /* notebook's "top 1%" of 128.  > 0 needs G = 32   */
    int64_t max_tokens;   /* capacity per stream, >= 1                        */
} kivi_config;

typedef struct kivi_cache kivi_cache;   /* opaque host-side handle */

/* Where everything sits inside the caller's device buffer (byte offsets from
   its start).  Packed blocks: [B*H][max_groups][block_bytes], block j of a
   stream holding tokens [32j, 32j+32) whatever G is.  At G = 32, inside a
   block (offsets below are from the block start): K codes, V codes
   (code_bytes = b*32*D/8 each), then fp16 K scale[D], K zero[D] of the key
   group, V scale[4][32], V zero[4][32]: slot cg of token t holds the
   parameters of the value group of channels 32cg .. 32cg+31.  With
   key_outliers = n > 0 (outlier-aware keys, the cookbook notebook's
   "Exercises" item 2, read per key group), the n channels of each key
   group with the largest max |K| over its tokens (ties: lower channel)
   keep their values in fp16: their codes, K scale and K zero in the block
   are 0, and the block's 256-byte record holds uint16 channel[3]
   (ascending, 0xFFFF unused), 10 zero bytes, then fp16 values [3][32] at
   byte 16 + 64 o (0 unused), then 48 zero bytes.
   Bit order of a code area (the storage cost, b bits per code and two fp16
   per group, is the notebook's storage cell; the order is this library's,
   chosen so that each lane's bytes are its own matrix-core operands): as
   little-endian uint32 dwords, lane l (0..63) and lane dword w (0..2b-1)
   name dword (w/4)*256 + 4l + w%4.  Its bits [16h + b i, 16h + b i + b)
   (half h = 0, 1; slot i = 0 .. 16/b - 1) hold the code at operand o,
   position kk:  b = 2, 4: o = w*(4/b) + i/4, kk = 2(i%4) + h;
                 b = 8:    o = w/2,         kk = 4(w%2) + 2i + h.
   Keys:   token 16(o/4) + l%16, channel 32(o%4) + 8(l/16) + kk.
   Values: token 4(l/16) + kk%4 + 16(kk/4), channel 16o + l%16.
   (Tokens are counted from the start of the block.)
   Split layout (G = 64 or 128, and the segment policy, whose value groups
   span all D channels): a block holds K codes, V codes, then fp16 V
   scale[D/G][32] and V zero[D/G][32] only (slot gv of token t: value group
   gv; off_vscale / off_vzero give the offsets), and the key zero / scale
   live once per key unit in the region at `kside`: [B*H][max_kside_units]
   units of fp16 K scale[D] then K zero[D] (off_kscale, off_kzero are the
   offsets inside a unit), unit u holding key group u (kside_unit_tokens =
   G tokens; the segment policy: one unit per 32-token block, the pair of
   the segment the block lies in).  The packed bytes are then exactly b bits
   per code and two fp16 per group ([NB] storage cell).
   Ring: [B*H][ring_capacity][D] in kv_dtype for K and for
   V; token t of a stream lives in slot t mod ring_capacity while it is in
   [G * floor(n_vquantized / G), n_tokens), which holds the key residual
   [n_quantized, n_tokens) and the value residual [n_vquantized, n_tokens). */
typedef struct {
    size_t blocks, ring_k, ring_v;      /* region offsets                     */
    size_t block_bytes, code_bytes;
    size_t off_kcode, off_vcode, off_kscale, off_kzero, off_vscale, off_vzero;
    int64_t max_groups;
    int64_t ring_capacity;              /* R + G                              */
    int64_t n_tokens;                   /* n                                  */
    int64_t n_quantized;                /* key tokens quantized: Q(n) / Q_K(n) */
    int64_t n_vquantized;               /* value tokens quantized: Q(n) / Q_V(n) */
    size_t outliers;                    /* key_outliers > 0: offset of the    */
                                        /* records [B*H][max_groups][256]     */
    size_t kside;                       /* split layout: offset of the key    */
                                        /*   units (0 otherwise)              */
    int64_t kside_unit_tokens;          /* tokens per key unit (0: in-block)  */
    int64_t max_kside_units;            /* key units per stream               */
} kivi_layout;

/* What an append of n_new tokens will do (pure host computation). */
typedef struct {
    int64_t n_old, n_new_total;         /* n before / after                   */
    int64_t q_old, q_new;               /* key prefix before / after          */
    int64_t flush_token_begin;          /* keys of tokens [q_old, q_new) are  */
    int64_t flush_token_end;            /*   quantized (t < n_old from ring)  */
    int64_t ring_token_begin;           /* tokens [max(G floor(v_flush_token_ */
    int64_t ring_token_end;             /*   end / G), n_old), n) -> the ring  */
    int64_t v_flush_token_begin;        /* values of tokens [qv_old, qv_new)  */
    int64_t v_flush_token_end;          /*   are quantized (= the key range   */
                                        /*   under the window policy)         */
} kivi_append_plan;

/* Bytes of device memory a cache with this config needs (0 if the config is
   invalid or unsupported): the packed blocks of max_tokens / 32 token
   groups per stream at b bits per code plus two fp16 per key and per value
   group (the notebook's storage cell: "2 fp16 per group"), and the two
   full-precision rings of R + G tokens ("KIVI", VeloxQuant-MLX docs, "How it
   works" item 3). */
size_t kivi_cache_bytes(const kivi_config *cfg);

/* Validate cfg and bind a host handle to the caller's device buffer
   (dev_mem, dev_bytes >= kivi_cache_bytes(cfg), 256-byte aligned).  The
   config is the method's: b-bit codes with G-element groups, keys per
   channel and values per token (notebook, "K (per-channel) and V
   (per-token) quantisation"; VeloxQuant-MLX docs, "How it works" items 1-2),
   and R full-precision tokens (item 3).  The
   cache starts empty; the buffer's contents need no initialization.  The
   buffer must outlive the handle.  *out is set only on KIVI_OK. */
kivi_status kivi_cache_create(const kivi_config *cfg, void *dev_mem,
                              size_t dev_bytes, kivi_cache **out);

/* Release the host handle (the device buffer is the caller's). NULL is ok. */
kivi_status kivi_cache_destroy(kivi_cache *c);

/* Append n_new >= 0 tokens to every stream ("KIVI", VeloxQuant-MLX docs,
   "How it works" items 3-4: the newest R tokens stay in full precision and
   older ones are quantized in whole groups of G; under KIVI_FLUSH_PAPER,
   "[Paper review] KIVI ...", 3.2.3 Algorithm 1, decoding phase).
   k, v: device, contiguous
   [B][H][n_new][D] in kv_dtype (may be NULL when n_new == 0); they are read
   by kernels enqueued on `stream` and must stay valid until those finish.
   Enqueues, in this order: quantization of the newly aged tokens (see
   kivi_append_plan: K per channel in whole groups, V per token; token t <
   n_old is read from the ring, later tokens from k/v), then the copy of the
   plan's ring range into the ring.  flags: 0 or KIVI_DEFER_FLUSH (then only
   the ring copy of [n_old, n) is enqueued and the quantized prefixes are
   left as they were).  Errors: INVALID_ARG (null handle, null k/v with
   n_new > 0, n_new < 0, unknown flags), CAPACITY (n + n_new > max_tokens;
   with KIVI_DEFER_FLUSH also when the ring would overflow, see above), HIP. */
kivi_status kivi_append(kivi_cache *c, const void *k, const void *v,
                        int64_t n_new, uint32_t flags, hipStream_t stream);

/* Make the cache canonical: quantize the tokens that deferred appends left
   in the ring up to the policy's prefixes (nothing to do after appends
   without KIVI_DEFER_FLUSH), in whole groups ("KIVI", VeloxQuant-MLX docs,
   "How it works" items 3-4).  Idempotent.  Errors: INVALID_ARG, HIP. */
kivi_status kivi_flush(kivi_cache *c, hipStream_t stream);

/* Host-only: what kivi_append(c, ..., n_new, 0, ...) would enqueue. */
kivi_status kivi_plan_append(const kivi_cache *c, int64_t n_new,
                             kivi_append_plan *out);

/* Workspace bytes kivi_decode_attn needs for any n <= max_tokens. */
size_t kivi_decode_workspace_bytes(const kivi_cache *c);

/* How decode splits the quantized prefix at the current n: *splits work
   items per stream over the groups with key and value codes,
   *groups_per_split groups each (plus one item per stream for the
   full-precision residual and, under the paper policy, one for the groups
   whose value codes stop inside or before them). Host-only. */
kivi_status kivi_decode_plan(const kivi_cache *c, int32_t *splits,
                             int32_t *groups_per_split);

/* One decode-attention step over all n cached tokens of every stream
   ("[Paper review] KIVI ...", 1.3 decoding: A = softmax(q K^T / sqrt(D)),
   o = A V; 3.2, dequantization fused into the two products):
   out[b][hq][:] = softmax(scale * q[b][hq] . K_hat^T) V_hat, where K_hat and
   V_hat are the dequantized tokens (code * scale + zero) followed by the
   full-precision residual (under the paper policy the key and value
   residuals differ), and query head hq reads KV head hq / (Hq / H).
   q: device [B][Hq][D] in q_dtype; out: device float32 [B][Hq][D];
   softmax_scale <= 0 selects 1/sqrt(D); workspace: device, ws_bytes >=
   kivi_decode_workspace_bytes(c).  Errors: INVALID_ARG (null pointers, bad
   q_dtype), STATE (n == 0, or a deferred flush pending: q < Q(n)),
   BUFFER_TOO_SMALL, HIP. */
kivi_status kivi_decode_attn(kivi_cache *c, const void *q, int32_t q_dtype,
                             float softmax_scale, float *out, void *workspace,
                             size_t ws_bytes, hipStream_t stream);

/* Bytes of the fixed device array kivi_decode_attn_noalloc keeps its decode
   partials in (one copy per device, held until the process ends). */
#define KIVI_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/* kivi_decode_attn without a workspace, for callers that cannot allocate
   device memory (code under HIP graph capture, allocation-free serving
   loops, harnesses that forbid hipMalloc).  Same arguments, results and
   kernels as kivi_decode_attn; the split partials go to a fixed device
   array of KIVI_NOALLOC_SCRATCH_BYTES inside the library instead of a
   caller workspace.  The call itself allocates nothing (the array's device
   address is looked up on the first call on each device).  Every call on a
   device shares that device's array: calls that overlap on one device (on
   different streams, or from different threads) race and must be ordered
   by the caller; nothing in the array needs to start at zero.  Errors:
   those of kivi_decode_attn, and BUFFER_TOO_SMALL when this cache's
   partials, kivi_decode_workspace_bytes(c), exceed
   KIVI_NOALLOC_SCRATCH_BYTES (B * Hq * items * (D + 2) * 4 bytes: 9.6 MB
   at batch 16 and 10.6 MB at batch 32 with 8 KV and 32 query heads,
   R = 128). */
kivi_status kivi_decode_attn_noalloc(kivi_cache *c, const void *q, int32_t q_dtype,
                                     float softmax_scale, float *out, hipStream_t stream);

/* kivi_append(c, k, v, n_new, 0, stream) followed by kivi_decode_attn(c, q,
   q_dtype, softmax_scale, out, workspace, ws_bytes, stream), with the same
   results bit for bit, for a serving loop's decode step ("[Paper review]
   KIVI ...", 1.3: append the new K/V, then attend).  When the append
   quantizes nothing (window policy, no group ages out: 31 of 32 single-token
   steps at G = 32), the new rows are not copied into the ring by a kernel
   of their own: the decode's residual items read them from k / v and write
   them into the ring, so k / v must stay valid until the decode finishes.
   Otherwise the call enqueues exactly what the two calls would.  Arguments
   as for the two calls (n_new >= 0; k, v may be NULL when n_new == 0).
   Everything is validated before anything is enqueued.  Errors: those of
   kivi_append (KIVI_DEFER_FLUSH is not accepted here) and of
   kivi_decode_attn; STATE also when a deferred flush is pending before the
   call.  HIP: if the append enqueues launches of its own (some group ages
   out, n_new == 0 or the paper policy) and the decode launch is the one
   refused, the append has taken effect exactly as a successful kivi_append
   and out is not written; otherwise the call had no effect. */
kivi_status kivi_append_decode(kivi_cache *c, const void *k, const void *v, int64_t n_new,
                               const void *q, int32_t q_dtype, float softmax_scale,
                               float *out, void *workspace, size_t ws_bytes,
                               hipStream_t stream);

/* Attention of T queries per (batch, query head) over all n cached tokens
   (the dequantized groups followed by the full-precision residual):
   out[b][hq][t][:] = softmax(scale * q[b][hq][t] . K_hat^T + mask) V_hat, the
   notebook's attention over every row of Q ("Attention output: quantised vs
   fp16" in [NB]).  causal = 0: every query sees all n tokens.  causal = 1:
   the queries are the last T cached tokens (appended before the call, as in
   [RV] 1.3), so query t sees tokens 0 .. n - T + t; needs T <= n.  T = 1
   without the mask is the decode step.  Query head hq reads KV head
   hq / (Hq / H).  With outlier-aware keys, K_hat of a key group's kept
   channels is their fp16 value from the block's record.
   q: device [B][Hq][T][D] in q_dtype; out: device float32 [B][Hq][T][D];
   softmax_scale <= 0 selects 1/sqrt(D); workspace: device, ws_bytes >=
   kivi_attn_workspace_bytes(c, T) (may be 0, then workspace may be NULL).
   Errors: INVALID_ARG (null pointers, T < 1, bad q_dtype or causal, causal
   with T > n), STATE (n == 0 or a deferred flush pending), UNSUPPORTED
   (B * Hq * T >= 2^31), BUFFER_TOO_SMALL, HIP.  Under the paper policy keys
   are the codes below Q_K and values the codes below Q_V, the ring's rows
   above each.  The products run on fp16 operands: rows of a float32 ring
   enter them rounded to nearest fp16 (finite up to 65504 in magnitude, as
   the fp16 zero / scale of the coded groups are). */
kivi_status kivi_attn(kivi_cache *c, const void *q, int32_t q_dtype, int64_t T,
                      int32_t causal, float softmax_scale, float *out,
                      void *workspace, size_t ws_bytes, hipStream_t stream);

/* Workspace bytes kivi_attn needs for T queries at any n <= max_tokens
   (0: none needed).  0 also for a null cache or T < 1. */
size_t kivi_attn_workspace_bytes(const kivi_cache *c, int64_t T);

/* How kivi_attn splits the work at the current n: *qblocks query blocks per
   stream (8 x 16/GQ queries each), *splits ranges of *groups_per_split
   groups (the last also walks the residual).  Host-only. */
kivi_status kivi_attn_plan(const kivi_cache *c, int64_t T, int32_t *qblocks,
                           int32_t *splits, int32_t *groups_per_split);

/* Offsets, sizes and the current n / Q(n) (host-only): where the packed
   codes and the fp16 zero / scale pairs of the notebook's storage cell, and
   the full-precision residual, sit in the caller's buffer (layout above). */
kivi_status kivi_get_layout(const kivi_cache *c, kivi_layout *out);

/* Static string for a status code. */
const char *kivi_status_string(kivi_status s);

#ifdef __cplusplus
}
#endif
#endif /* KIVI_H */
