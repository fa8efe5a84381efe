/*
 * kivi_oracle.c -- plain, slow, scalar CPU reference for KIVI KV-cache
 * quantization and decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or
 * calls this file: only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark do.  It shares no code, header, table or constant with the
 * HIP library; it is written from the pages' definitions, one step at a time,
 * in the pages' order, so that a reader can check it by eye.
 *
 * Sources (cited by page title and section):
 *  [NB]  "KIVI - 2-bit KV cache quantisation" (LLM systems cookbook, serving
 *        notebook 04): sections "Asymmetric 2-bit quantiser", "K
 *        (per-channel) and V (per-token) quantisation", "Attention output:
 *        quantised vs fp16", storage cell.
 *  [VQ]  "KIVI" (VeloxQuant-MLX algorithm docs): "How it works" items 1-4 and
 *        the zero/scale/q/recon formulas; "Re-measured after #162".
 *  [RV]  "[Paper review] KIVI: A Tuning-Free Asymmetric 2bit Quantization for
 *        KV Cache (ICML'24)" (chooblog): 1.1 quantization definition and its
 *        worked example; 1.3 inference workflow; 3.2.2 grouped + residual
 *        split; 3.2.3 Algorithm 1 (prefill / decoding) and its example.
 *  [CQ]  "KV Cache Compression > Cache Quantization" (Language AI Handbook):
 *        uniform quantization, the half-step error bound, QuantizedCache.
 *  [GR]  GEAR paper review (velog): "KCVT" (KIVI's coarse-grained grouping)
 *        and "streaming buffer strategy".
 *
 * Parity status: every function is pinned by tests/test_oracle_pins.py to
 * what the pages print or to closed forms.  The packers (oracle_pack_blocks_kv
 * in both layouts, with the key units of the split layout,
 * oracle_pack_outlier_records) are pinned by tests/test_oracle_layout_pins.py,
 * which decodes their output with its own forward reading of the documented
 * byte layout (never through code_position) back to the pinned logical
 * arrays, the paper-policy zero rows included.  The KCVT segment builder is
 * pinned by tests/test_oracle_kcvt_pins.py (reductions to pinned KIVI group
 * sizes, closed-form statistics, locality, the documented block layout).  The bit order itself is a
 * layout choice of this library: the pages fix the storage cost (b bits per
 * code and two fp16 per group), not the order.
 *
 * Build: gcc -O2 -fno-fast-math -ffp-contract=off -fPIC -shared
 * (x86-64 SSE arithmetic: every float operation below is one IEEE-754
 * binary32 operation rounded to nearest even; no FMA contraction.)
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* IEEE-754 binary16 <-> binary32, written from the format definition.       */
/* The cache stores zero and scale as fp16 ([NB] storage cell: "2 fp16 per   */
/* group").  Rounding is to nearest, ties to even; subnormals are kept;      */
/* magnitudes that round past 65504 become infinity.                         */
/* ------------------------------------------------------------------------ */

float oracle_f16_to_f32(uint16_t h)
{
    uint32_t sign = (uint32_t)(h >> 15) & 1u;
    uint32_t e = (uint32_t)(h >> 10) & 0x1Fu;
    uint32_t m = (uint32_t)h & 0x3FFu;
    double v;
    if (e == 0x1F) {
        if (m != 0) return NAN;
        v = INFINITY;
    } else if (e == 0) {
        v = ldexp((double)m, -24);                 /* subnormal: m * 2^-24 */
    } else {
        v = ldexp((double)(m | 0x400u), (int)e - 25);   /* (1024+m) * 2^(e-25) */
    }
    return (float)(sign ? -v : v);                 /* exact: fits binary32 */
}

uint16_t oracle_f32_to_f16(float f)
{
    uint32_t x;
    memcpy(&x, &f, 4);
    uint16_t sign = (uint16_t)((x >> 16) & 0x8000u);
    uint32_t be = (x >> 23) & 0xFFu;
    uint32_t man = x & 0x7FFFFFu;
    if (be == 0xFF) return (uint16_t)(sign | 0x7C00u | (man ? 0x200u : 0u));
    if (be == 0) return sign;      /* |f| < 2^-126: far below half of 2^-24 */
    /* |f| = m24 * 2^(be-150) with m24 in [2^23, 2^24). */
    uint32_t m24 = man | 0x800000u;
    int E = (int)be - 127;                          /* unbiased exponent */
    int qe = (E > -14 ? E : -14) - 10;              /* fp16 quantum 2^qe */
    int sh = qe - ((int)be - 150);                  /* >= 13 */
    uint32_t r;
    if (sh >= 25) {
        r = 0;                                      /* below half a quantum */
    } else {
        uint32_t keep = m24 >> sh;
        uint32_t rem = m24 & ((1u << sh) - 1u);
        uint32_t half = 1u << (sh - 1);
        r = keep;
        if (rem > half || (rem == half && (keep & 1u))) r++;
    }
    /* value = r * 2^qe; encode. For E <= -14 the bits are r itself
       (r == 1024 is the smallest normal); above, the exponent field
       follows E and a carry to r == 2048 rolls into the next binade. */
    uint32_t bits = (E > -14) ? ((uint32_t)(E + 14) << 10) + r : r;
    if (bits >= 0x7C00u) bits = 0x7C00u;
    return (uint16_t)(sign | bits);
}

/* Round half to even ([NB] uses torch.round, which rounds ties to even). */
static float round_half_even(float t)
{
    float f = floorf(t);
    float r = t - f;                /* exact for |t| < 2^23 */
    if (r > 0.5f) return f + 1.0f;
    if (r < 0.5f) return f;
    return (fmodf(f, 2.0f) == 0.0f) ? f : f + 1.0f;
}

/* ------------------------------------------------------------------------ */
/* GroupQuant: asymmetric min/max quantization of one group.                 */
/* [NB] "Asymmetric 2-bit quantiser"; [VQ] "How it works" formulas;          */
/* [RV] 1.1:  z = min X,  s = (max X - min X) / (2^B - 1),                   */
/*            Q(X) = round((X - z) / s),  X' = Q(X) * s + z.                 */
/* Guard for a constant group: s == 0 -> s = 1 ([NB] quantiser, [CQ]).       */
/* Codes are computed from the float32 (z, s); the stored pair is            */
/* (fp16(z), fp16(s)).                                                       */
/* ------------------------------------------------------------------------ */
void oracle_group_quant(const float *g, int n, int bits, uint8_t *codes,
                        float *mn_out, float *s_out,
                        uint16_t *zero16, uint16_t *scale16)
{
    const float L = (float)((1 << bits) - 1);
    float mn = g[0], mx = g[0];
    for (int i = 1; i < n; i++) {
        if (g[i] < mn) mn = g[i];
        if (g[i] > mx) mx = g[i];
    }
    if (mn == 0.0f) mn = 0.0f;          /* a zero minimum is stored as +0 */
    float rng = mx - mn;
    float s = rng / L;
    if (s == 0.0f) s = 1.0f;
    for (int i = 0; i < n; i++) {
        float d = g[i] - mn;
        float t = d / s;
        float c = round_half_even(t);
        if (c < 0.0f) c = 0.0f;
        if (c > L) c = L;
        codes[i] = (uint8_t)c;
    }
    if (mn_out) *mn_out = mn;
    if (s_out) *s_out = s;
    if (zero16) *zero16 = oracle_f32_to_f16(mn);
    if (scale16) *scale16 = oracle_f32_to_f16(s);
}

/* Dequantization of one code with the stored fp16 pair:
   x_hat = code * scale + zero, two float32 roundings ([VQ] recon formula). */
float oracle_dequant_one(uint8_t code, uint16_t zero16, uint16_t scale16)
{
    float p = (float)code * oracle_f16_to_f32(scale16);
    return p + oracle_f16_to_f32(zero16);
}

/* ------------------------------------------------------------------------ */
/* Flush policies: how many tokens of an n-token stream are quantized.       */
/* Window policy ([VQ] items 3-4): the newest R tokens stay fp16 and aged    */
/* tokens are quantized only in whole multiples of G, for K and V alike:     */
/*        Q(n) = G * floor(max(0, n - R) / G).                               */
/* Paper policy ([RV] 3.2.2 / 3.2.3 Algorithm 1): keys keep r = n mod R      */
/* tokens in full precision (Q_K = n - r); values keep the newest R          */
/* (Q_V = max(0, n - R)).                                                    */
/* ------------------------------------------------------------------------ */
/* Segment policy (KCVT, the GEAR review's "KCVT" and "streaming buffer     */
/* strategy" sections): new tokens wait in a full-precision buffer of R      */
/* tokens and are compressed when it fills, keys and values alike:           */
/*        Q(n) = n - (n mod R).                                              */
enum { ORACLE_POLICY_WINDOW = 0, ORACLE_POLICY_PAPER = 1, ORACLE_POLICY_SEGMENT = 2 };

void oracle_quantized_prefix(int64_t n, int group, int residual, int policy,
                             int64_t *qk, int64_t *qv)
{
    if (policy == ORACLE_POLICY_SEGMENT) {
        *qk = *qv = n - (n % residual);
    } else if (policy == ORACLE_POLICY_PAPER) {
        /* R > 0 required by the paper's definition r = l mod R. */
        *qk = n - (n % residual);
        *qv = n > residual ? n - residual : 0;
    } else {
        int64_t aged = n > residual ? n - residual : 0;
        *qk = *qv = (aged / group) * group;
    }
}

static float load_elem(const void *x, int dtype, int64_t idx)
{
    if (dtype == 0) return oracle_f16_to_f32(((const uint16_t *)x)[idx]);
    return ((const float *)x)[idx];
}

/* ------------------------------------------------------------------------ */
/* Build the logical cache of one layer from n tokens.                       */
/* Inputs k, v: [B][H][n][D] in dtype (0 = fp16 bits, 1 = float32).          */
/* Keys per channel: group (b,h,j,c) = K[b,h, jG..jG+G-1, c]  ([NB] K along  */
/* dim 0, [VQ] item 1, [RV] 3.2.3 step D).                                   */
/* Values per token: group (b,h,t,j) = V[b,h,t, jG..jG+G-1]  ([NB] V along   */
/* dim 1, [VQ] item 2, [RV] 3.2.3 step C).                                   */
/* Outputs (logical, unpacked):                                              */
/*   kcodes [B][H][qk][D] u8,  kzero16/kscale16 [B][H][qk/G][D]              */
/*   vcodes [B][H][qv][D] u8,  vzero16/vscale16 [B][H][qv][D/G]              */
/* where qk, qv come from oracle_quantized_prefix (caller passes them).      */
/* ------------------------------------------------------------------------ */
void oracle_build_cache(const void *k, const void *v, int dtype,
                        int B, int H, int64_t n, int D, int G, int bits,
                        int64_t qk, int64_t qv,
                        uint8_t *kcodes, uint16_t *kzero16, uint16_t *kscale16,
                        uint8_t *vcodes, uint16_t *vzero16, uint16_t *vscale16)
{
    float *grp = (float *)malloc(sizeof(float) * (size_t)G);
    uint8_t *cg = (uint8_t *)malloc((size_t)G);
    for (int b = 0; b < B; b++)
        for (int h = 0; h < H; h++) {
            int64_t base = ((int64_t)b * H + h) * n * D;
            /* keys: per channel, G consecutive tokens */
            for (int64_t j = 0; j < qk / G; j++)
                for (int c = 0; c < D; c++) {
                    for (int i = 0; i < G; i++)
                        grp[i] = load_elem(k, dtype, base + (j * G + i) * D + c);
                    int64_t pidx = (((int64_t)b * H + h) * (qk / G) + j) * D + c;
                    oracle_group_quant(grp, G, bits, cg, NULL, NULL,
                                       &kzero16[pidx], &kscale16[pidx]);
                    for (int i = 0; i < G; i++)
                        kcodes[(((int64_t)b * H + h) * qk + j * G + i) * D + c] = cg[i];
                }
            /* values: per token, G consecutive channels */
            for (int64_t t = 0; t < qv; t++)
                for (int j = 0; j < D / G; j++) {
                    for (int i = 0; i < G; i++)
                        grp[i] = load_elem(v, dtype, base + t * D + j * G + i);
                    int64_t pidx = (((int64_t)b * H + h) * qv + t) * (D / G) + j;
                    oracle_group_quant(grp, G, bits, cg, NULL, NULL,
                                       &vzero16[pidx], &vscale16[pidx]);
                    for (int i = 0; i < G; i++)
                        vcodes[(((int64_t)b * H + h) * qv + t) * D + j * G + i] = cg[i];
                }
        }
    free(grp);
    free(cg);
}

/* ------------------------------------------------------------------------ */
/* KCVT: the coarse-grained grouping of the GEAR review ("KCVT" section).    */
/* Keys are quantized per channel with one group per channel over all the    */
/* tokens compressed together, values per token with one group over all D    */
/* channels.  With the streaming buffer ("streaming buffer strategy"         */
/* section) the tokens compressed together are those of one flush: the whole */
/* prompt at prefill, then each buffer of new tokens.  Reading taken here:   */
/* segment i is tokens [seg_end[i-1], seg_end[i]) (seg_end[-1] = 0), every   */
/* boundary a multiple of 32; the key group of (segment i, channel c) is     */
/* K[seg_end[i-1] .. seg_end[i]-1][c].  Q = seg_end[n_seg-1] tokens are      */
/* quantized.  Outputs:                                                      */
/*   kcodes [B][H][Q][D] u8; kzero16 / kscale16 [B][H][Q/32][D]: the pair of */
/*   the segment each 32-token block lies in (repeated over its blocks);     */
/*   vcodes [B][H][Q][D] u8; vzero16 / vscale16 [B][H][Q][1].                */
/* ------------------------------------------------------------------------ */
void oracle_build_cache_segments(const void *k, const void *v, int dtype,
                                 int B, int H, int64_t n, int D, int bits,
                                 const int64_t *seg_end, int n_seg,
                                 uint8_t *kcodes, uint16_t *kzero16, uint16_t *kscale16,
                                 uint8_t *vcodes, uint16_t *vzero16, uint16_t *vscale16)
{
    const int T = 32;
    int64_t Q = n_seg > 0 ? seg_end[n_seg - 1] : 0;
    int64_t longest = D;
    for (int i = 0; i < n_seg; i++) {
        int64_t a = i ? seg_end[i - 1] : 0;
        if (seg_end[i] - a > longest) longest = seg_end[i] - a;
    }
    float *grp = (float *)malloc(sizeof(float) * (size_t)longest);
    uint8_t *cg = (uint8_t *)malloc((size_t)longest);
    for (int64_t s = 0; s < (int64_t)B * H; s++) {
        int64_t base = s * n * D;
        /* keys: one group per (segment, channel) */
        for (int i = 0; i < n_seg; i++) {
            int64_t a = i ? seg_end[i - 1] : 0, e = seg_end[i];
            int len = (int)(e - a);
            for (int c = 0; c < D; c++) {
                for (int t = 0; t < len; t++)
                    grp[t] = load_elem(k, dtype, base + (a + t) * D + c);
                uint16_t z16, s16;
                oracle_group_quant(grp, len, bits, cg, NULL, NULL, &z16, &s16);
                for (int t = 0; t < len; t++) kcodes[(s * Q + a + t) * D + c] = cg[t];
                for (int64_t j = a / T; j < e / T; j++) {
                    kzero16[(s * (Q / T) + j) * D + c] = z16;
                    kscale16[(s * (Q / T) + j) * D + c] = s16;
                }
            }
        }
        /* values: one group per token over all D channels */
        for (int64_t t = 0; t < Q; t++) {
            for (int c = 0; c < D; c++) grp[c] = load_elem(v, dtype, base + t * D + c);
            oracle_group_quant(grp, D, bits, cg, NULL, NULL, &vzero16[s * Q + t],
                               &vscale16[s * Q + t]);
            for (int c = 0; c < D; c++) vcodes[(s * Q + t) * D + c] = cg[c];
        }
    }
    free(grp);
    free(cg);
}

/* ------------------------------------------------------------------------ */
/* Outlier-aware keys ([NB] "Exercises" item 2: keep the top 1% of K         */
/* channels at fp16 and quantize the rest).  Reading taken here: within each */
/* key group (G tokens of a stream), the n_out channels with the largest     */
/* max |K| over the group's tokens (ties: the lower channel index) keep      */
/* their values, rounded to fp16; their codes, zero and scale are stored as  */
/* 0, so that code * scale + zero contributes nothing.  Selection per group  */
/* keeps the cache independent of how the tokens were chunked.  Applied to   */
/* the arrays oracle_build_cache wrote for the same inputs and qk.           */
/*   kout_idx [B*H][qk/G][n_out]  int32, ascending channel indices           */
/*   kout_val [B*H][qk/G][n_out][G] fp16 bits                                */
/* ------------------------------------------------------------------------ */
void oracle_key_outliers(const void *k, int dtype, int B, int H, int64_t n, int D, int G,
                         int64_t qk, int n_out, uint8_t *kcodes, uint16_t *kzero16,
                         uint16_t *kscale16, int32_t *kout_idx, uint16_t *kout_val)
{
    float *score = (float *)malloc(sizeof(float) * (size_t)D);
    int *chosen = (int *)malloc(sizeof(int) * (size_t)D);
    for (int64_t s = 0; s < (int64_t)B * H; s++) {
        int64_t base = s * n * D;
        for (int64_t j = 0; j < qk / G; j++) {
            /* max |K| of every channel over the group's tokens */
            for (int c = 0; c < D; c++) {
                float m = 0.0f;
                for (int i = 0; i < G; i++) {
                    float a = fabsf(load_elem(k, dtype, base + (j * G + i) * D + c));
                    if (a > m) m = a;
                }
                score[c] = m;
                chosen[c] = 0;
            }
            /* the n_out largest, one at a time (strictly larger wins: ties
               keep the lower channel index) */
            for (int o = 0; o < n_out; o++) {
                int best = -1;
                for (int c = 0; c < D; c++)
                    if (!chosen[c] && (best < 0 || score[c] > score[best])) best = c;
                chosen[best] = 1;
            }
            int o = 0;
            for (int c = 0; c < D; c++) {
                if (!chosen[c]) continue;
                int64_t g = s * (qk / G) + j;
                kout_idx[g * n_out + o] = c;
                for (int i = 0; i < G; i++) {
                    float x = load_elem(k, dtype, base + (j * G + i) * D + c);
                    kout_val[(g * n_out + o) * G + i] = oracle_f32_to_f16(x);
                    kcodes[(s * qk + j * G + i) * D + c] = 0;
                }
                kzero16[g * D + c] = 0;
                kscale16[g * D + c] = 0;
                o++;
            }
        }
    }
    free(score);
    free(chosen);
}

/* K-hat of the outlier channels: their stored fp16 values (the other
   channels keep what oracle_dequant_cache wrote).  khat [B][H][n][D]. */
void oracle_apply_key_outliers(int B, int H, int64_t n, int D, int G, int64_t qk, int n_out,
                               const int32_t *kout_idx, const uint16_t *kout_val, float *khat)
{
    for (int64_t s = 0; s < (int64_t)B * H; s++)
        for (int64_t j = 0; j < qk / G; j++)
            for (int o = 0; o < n_out; o++) {
                int64_t g = s * (qk / G) + j;
                int c = kout_idx[g * n_out + o];
                for (int i = 0; i < G; i++)
                    khat[(s * n + j * G + i) * D + c] =
                        oracle_f16_to_f32(kout_val[(g * n_out + o) * G + i]);
            }
}

/* ------------------------------------------------------------------------ */
/* Dequantized view of the whole cache ([RV] 1.1 X' = Q(X) s + z; tokens in  */
/* the full-precision residual are taken as they are, converted to float).   */
/* khat, vhat: [B][H][n][D] float32.                                         */
/* ------------------------------------------------------------------------ */
/* Key parameters per Gk tokens, value parameters per Gv channels (the      */
/* per-group arrays of oracle_build_cache have Gk = Gv = G; those of         */
/* oracle_build_cache_segments have Gk = 32, Gv = D).                        */
void oracle_dequant_cache_kv(const void *k, const void *v, int dtype,
                             int B, int H, int64_t n, int D, int Gk, int Gv,
                             int64_t qk, int64_t qv,
                             const uint8_t *kcodes, const uint16_t *kzero16,
                             const uint16_t *kscale16,
                             const uint8_t *vcodes, const uint16_t *vzero16,
                             const uint16_t *vscale16,
                             float *khat, float *vhat)
{
    for (int b = 0; b < B; b++)
        for (int h = 0; h < H; h++) {
            int64_t s = (int64_t)b * H + h;
            for (int64_t t = 0; t < n; t++)
                for (int c = 0; c < D; c++) {
                    int64_t o = (s * n + t) * D + c;
                    if (t < qk) {
                        int64_t p = (s * (qk / Gk) + t / Gk) * D + c;
                        khat[o] = oracle_dequant_one(kcodes[(s * qk + t) * D + c],
                                                     kzero16[p], kscale16[p]);
                    } else {
                        khat[o] = load_elem(k, dtype, o);
                    }
                    if (t < qv) {
                        int64_t p = (s * qv + t) * (D / Gv) + c / Gv;
                        vhat[o] = oracle_dequant_one(vcodes[(s * qv + t) * D + c],
                                                     vzero16[p], vscale16[p]);
                    } else {
                        vhat[o] = load_elem(v, dtype, o);
                    }
                }
        }
}

void oracle_dequant_cache(const void *k, const void *v, int dtype,
                          int B, int H, int64_t n, int D, int G,
                          int64_t qk, int64_t qv,
                          const uint8_t *kcodes, const uint16_t *kzero16,
                          const uint16_t *kscale16,
                          const uint8_t *vcodes, const uint16_t *vzero16,
                          const uint16_t *vscale16,
                          float *khat, float *vhat)
{
    oracle_dequant_cache_kv(k, v, dtype, B, H, n, D, G, G, qk, qv, kcodes, kzero16, kscale16,
                            vcodes, vzero16, vscale16, khat, vhat);
}

/* ------------------------------------------------------------------------ */
/* Decode attention over a (dequantized) cache, fp64 accumulation.           */
/* [NB] attn: softmax(Q K^T / sqrt(D)) V ; [RV] 1.3 decoding step:           */
/* A = Softmax(t_Q X_K^T), t_O = A X_V.  Grouped-query attention: query      */
/* head hq reads KV head hq / (Hq / H).                                      */
/* q: [B][Hq][D] float32; khat, vhat: [B][H][n][D]; out: [B][Hq][D].         */
/* ------------------------------------------------------------------------ */
void oracle_decode_attn(const float *q, const float *khat, const float *vhat,
                        int B, int H, int Hq, int64_t n, int D, double sm_scale,
                        float *out)
{
    double *sc = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    double *acc = (double *)malloc(sizeof(double) * (size_t)D);
    int ratio = Hq / H;
    for (int b = 0; b < B; b++)
        for (int hq = 0; hq < Hq; hq++) {
            int h = hq / ratio;
            const float *qq = q + ((int64_t)b * Hq + hq) * D;
            const float *kk = khat + ((int64_t)b * H + h) * n * D;
            const float *vv = vhat + ((int64_t)b * H + h) * n * D;
            double m = -INFINITY;
            for (int64_t t = 0; t < n; t++) {
                double s = 0.0;
                for (int c = 0; c < D; c++) s += (double)qq[c] * (double)kk[t * D + c];
                sc[t] = s * sm_scale;
                if (sc[t] > m) m = sc[t];
            }
            double l = 0.0;
            for (int c = 0; c < D; c++) acc[c] = 0.0;
            for (int64_t t = 0; t < n; t++) {
                double p = exp(sc[t] - m);
                l += p;
                for (int c = 0; c < D; c++) acc[c] += p * (double)vv[t * D + c];
            }
            float *o = out + ((int64_t)b * Hq + hq) * D;
            for (int c = 0; c < D; c++) o[c] = (float)(acc[c] / l);
        }
    free(sc);
    free(acc);
}

/* ------------------------------------------------------------------------ */
/* Attention of T queries per (batch, query head) over a (dequantized)       */
/* cache, fp64 accumulation.  [NB] attn: every row of Q attends over all of  */
/* K, V (no mask).  causal = 1: the T queries are the last T cached tokens   */
/* (appended before the call, [RV] 1.3: append, then attend), so query t     */
/* sits at position n - T + t and sees tokens 0 .. n - T + t.                */
/* q: [B][Hq][T][D] float32; khat, vhat: [B][H][n][D]; out: [B][Hq][T][D].   */
/* ------------------------------------------------------------------------ */
void oracle_attn_queries(const float *q, const float *khat, const float *vhat,
                         int B, int H, int Hq, int64_t T, int64_t n, int D,
                         double sm_scale, int causal, float *out)
{
    double *sc = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    double *acc = (double *)malloc(sizeof(double) * (size_t)D);
    int ratio = Hq / H;
    for (int b = 0; b < B; b++)
        for (int hq = 0; hq < Hq; hq++) {
            int h = hq / ratio;
            const float *kk = khat + ((int64_t)b * H + h) * n * D;
            const float *vv = vhat + ((int64_t)b * H + h) * n * D;
            for (int64_t t = 0; t < T; t++) {
                const float *qq = q + (((int64_t)b * Hq + hq) * T + t) * D;
                int64_t seen = causal ? n - T + t + 1 : n;     /* tokens 0 .. seen-1 */
                double m = -INFINITY;
                for (int64_t j = 0; j < seen; j++) {
                    double s = 0.0;
                    for (int c = 0; c < D; c++) s += (double)qq[c] * (double)kk[j * D + c];
                    sc[j] = s * sm_scale;
                    if (sc[j] > m) m = sc[j];
                }
                double l = 0.0;
                for (int c = 0; c < D; c++) acc[c] = 0.0;
                for (int64_t j = 0; j < seen; j++) {
                    double p = exp(sc[j] - m);
                    l += p;
                    for (int c = 0; c < D; c++) acc[c] += p * (double)vv[j * D + c];
                }
                float *o = out + (((int64_t)b * Hq + hq) * T + t) * D;
                for (int c = 0; c < D; c++) o[c] = (float)(acc[c] / l);
            }
        }
    free(sc);
    free(acc);
}

/* ------------------------------------------------------------------------ */
/* Packed storage of one token group of one (batch, KV-head) stream.         */
/*                                                                           */
/* The pages fix the storage cost (b bits per code, two fp16 per group,      */
/* [NB] storage cell) but not the bit order.  This library's order puts,     */
/* for each 32-token x 128-channel tile, the codes one 64-lane wavefront     */
/* needs for a matrix-core operand into that lane's own 16 bytes:            */
/*                                                                           */
/*   block = [K codes | V codes | K scale[D] | K zero[D] |                   */
/*            V scale[D/G][G] | V zero[D/G][G]]    (codes: b*G*D/8 bytes)    */
/*                                                                           */
/* Code dword index (within one code area) for lane l (0..63), lane dword w  */
/* (0..2b-1): (w/4)*256 + 4*l + (w%4).  Inside a dword, the code of slot i   */
/* (0 <= i < 16/b) in half h (0,1) sits at bit 16*h + b*i and belongs to     */
/*   operand o = w*(4/b) + i/4,  kk = 2*(i%4) + h        (b = 2, 4)          */
/*   operand o = w/2,            kk = 4*(w%2) + 2*i + h  (b = 8: an operand  */
/*                               spans two dwords)                           */
/* Keys:   token = 16*(o/4) + l%16,      channel = 32*(o%4) + 8*(l/16) + kk  */
/* Values: channel = 16*o + l%16,        token = 4*(l/16) + kk%4 + 16*(kk/4) */
/* Only D = 128, G = 32 is laid out this way.                                */
/* ------------------------------------------------------------------------ */
static void code_position(int bits, int is_v, int token, int channel,
                          int64_t *dword, int *bit)
{
    /* Invert the mapping above by search: plain and obviously bijective. */
    int dpl = 2 * bits;
    for (int l = 0; l < 64; l++)
        for (int w = 0; w < dpl; w++)
            for (int h = 0; h < 2; h++)
                for (int i = 0; i < 16 / bits; i++) {
                    int o = bits == 8 ? w / 2 : w * (4 / bits) + i / 4;
                    int kk = bits == 8 ? 4 * (w % 2) + 2 * i + h : 2 * (i % 4) + h;
                    int t, c;
                    if (!is_v) {
                        t = 16 * (o / 4) + l % 16;
                        c = 32 * (o % 4) + 8 * (l / 16) + kk;
                    } else {
                        c = 16 * o + l % 16;
                        t = 4 * (l / 16) + kk % 4 + 16 * (kk / 4);
                    }
                    if (t == token && c == channel) {
                        *dword = (int64_t)(w / 4) * 256 + 4 * l + (w % 4);
                        *bit = 16 * h + bits * i;
                        return;
                    }
                }
    *dword = -1;
    *bit = -1;
}

int64_t oracle_block_bytes(int bits)
{
    const int D = 128, G = 32;
    return 2 * (int64_t)(bits * G * D / 8) + 4 * (int64_t)D * 2;
}

/* Bytes of one 32-token block when value groups span Gv channels: with
   Gv = 32 the block carries its key group's zero / scale and four value
   slots per token (oracle_block_bytes); with Gv > 32 (the split layout) it
   carries only the codes and its tokens' D / Gv value pairs, and the key
   zero / scale live once per key group in a separate array. */
int64_t oracle_block_bytes_g(int bits, int Gv)
{
    const int D = 128, T = 32;
    if (Gv == T) return oracle_block_bytes(bits);
    return 2 * (int64_t)(bits * T * D / 8) + 2 * 2 * (int64_t)T * (D / Gv);
}

/* Pack the quantized tokens of each stream into 32-token blocks:
   out [B*H][max_groups][oracle_block_bytes_g(bits, Gv)].  Keys of the first
   nk tokens (nk a multiple of Gk) and values of the first nv tokens, from
   the logical arrays of oracle_build_cache (Gk = Gv = G, G in {32, 64, 128})
   or oracle_build_cache_segments (Gk = 32, Gv = D): kcodes [B*H][nk][D],
   kzero16 / kscale16 [B*H][nk/Gk][D], vcodes [B*H][nv][D], vzero16 /
   vscale16 [B*H][nv][D/Gv].
   Gv = 32: a block holds K codes, V codes, then fp16 K scale[D], K zero[D]
   of the key group it lies in, V scale[4][32], V zero[4][32] (slot cg of
   token t: the value group of channels 32cg .. 32cg+31).
   Gv > 32 (split layout, two fp16 per group as the notebook's storage cell
   counts them): a block holds K codes, V codes, then fp16 V scale[D/Gv][32],
   V zero[D/Gv][32] (slot gv of token t: value group gv); key unit u (the
   key group of tokens [u Gk, u Gk + Gk)) of stream s is kside [B*H]
   [max_kunits][2][D]: K scale[D], then K zero[D].
   Every code or side entry of a token that is not quantized (a value row
   at or past nv inside a block that holds value rows) is 0; blocks and key
   units past the prefixes are left as they are.  kside may be NULL when
   Gv = 32. */
void oracle_pack_blocks_kv2(int B, int H, int Gk, int Gv, int64_t nk, int64_t nv, int bits,
                            int64_t max_groups, int64_t max_kunits,
                            const uint8_t *kcodes, const uint16_t *kzero16,
                            const uint16_t *kscale16,
                            const uint8_t *vcodes, const uint16_t *vzero16,
                            const uint16_t *vscale16, uint8_t *out, uint16_t *kside);

void oracle_pack_blocks_kv(int B, int H, int G, int64_t nk, int64_t nv, int bits,
                           int64_t max_groups, int64_t max_kunits,
                           const uint8_t *kcodes, const uint16_t *kzero16,
                           const uint16_t *kscale16,
                           const uint8_t *vcodes, const uint16_t *vzero16,
                           const uint16_t *vscale16, uint8_t *out, uint16_t *kside)
{
    oracle_pack_blocks_kv2(B, H, G, G, nk, nv, bits, max_groups, max_kunits, kcodes, kzero16,
                           kscale16, vcodes, vzero16, vscale16, out, kside);
}

void oracle_pack_blocks_kv2(int B, int H, int Gk, int Gv, int64_t nk, int64_t nv, int bits,
                            int64_t max_groups, int64_t max_kunits,
                            const uint8_t *kcodes, const uint16_t *kzero16,
                            const uint16_t *kscale16,
                            const uint8_t *vcodes, const uint16_t *vzero16,
                            const uint16_t *vscale16, uint8_t *out, uint16_t *kside)
{
    const int D = 128, T = 32;      /* channels; tokens per block */
    const int split = Gv > T;
    const int nvg = D / Gv;         /* value groups per token */
    const int64_t cbytes = bits * T * D / 8;
    const int64_t bb = oracle_block_bytes_g(bits, Gv);
    /* position tables for one tile, computed by the search above */
    int64_t *kd = (int64_t *)malloc(sizeof(int64_t) * T * D);
    int64_t *vd = (int64_t *)malloc(sizeof(int64_t) * T * D);
    int *kb = (int *)malloc(sizeof(int) * T * D);
    int *vb = (int *)malloc(sizeof(int) * T * D);
    for (int t = 0; t < T; t++)
        for (int c = 0; c < D; c++) {
            code_position(bits, 0, t, c, &kd[t * D + c], &kb[t * D + c]);
            code_position(bits, 1, t, c, &vd[t * D + c], &vb[t * D + c]);
        }
    int64_t ngk = nk / T;             /* blocks with key codes */
    int64_t ngv = (nv + T - 1) / T;   /* blocks with value rows */
    int64_t ng = ngk > ngv ? ngk : ngv;
    for (int64_t s = 0; s < (int64_t)B * H; s++) {
        for (int64_t j = 0; j < ng; j++) {
            uint8_t *blk = out + (s * max_groups + j) * bb;
            uint32_t *kc = (uint32_t *)blk;
            uint32_t *vc = (uint32_t *)(blk + cbytes);
            uint16_t *side = (uint16_t *)(blk + 2 * cbytes);
            uint16_t *vs = split ? side : side + 2 * D;
            uint16_t *vz = vs + (split ? nvg : D / T) * T;
            if (j < ngk) {
                /* key group of this block: tokens [jT, jT + T) lie in group jT / Gk */
                int64_t kg = (s * (nk / Gk) + (j * T) / Gk) * D;
                memset(kc, 0, (size_t)cbytes);
                for (int t = 0; t < T; t++)
                    for (int c = 0; c < D; c++) {
                        uint32_t ck = kcodes[(s * nk + j * T + t) * D + c];
                        kc[kd[t * D + c]] |= ck << kb[t * D + c];
                    }
                if (!split)
                    for (int c = 0; c < D; c++) {
                        side[c] = kscale16[kg + c];
                        side[D + c] = kzero16[kg + c];
                    }
            }
            if (j < ngv) {
                memset(vc, 0, (size_t)cbytes);
                for (int t = 0; t < T; t++) {
                    int64_t tok = j * T + t;
                    for (int c = 0; c < D; c++) {
                        uint32_t cv = tok < nv ? vcodes[(s * nv + tok) * D + c] : 0;
                        vc[vd[t * D + c]] |= cv << vb[t * D + c];
                    }
                    if (split) {
                        /* slot gv: value group gv */
                        for (int gv = 0; gv < nvg; gv++) {
                            int64_t vg = (s * nv + tok) * nvg + gv;
                            vs[gv * T + t] = tok < nv ? vscale16[vg] : 0;
                            vz[gv * T + t] = tok < nv ? vzero16[vg] : 0;
                        }
                    } else {
                        /* slot cg: channels 32cg .. 32cg+31, in value group 32cg / Gv */
                        for (int cg = 0; cg < D / T; cg++) {
                            int64_t vg = (s * nv + tok) * (D / Gv) + (cg * T) / Gv;
                            vs[cg * T + t] = tok < nv ? vscale16[vg] : 0;
                            vz[cg * T + t] = tok < nv ? vzero16[vg] : 0;
                        }
                    }
                }
            }
        }
        /* split layout: one key unit per key group */
        if (split && kside)
            for (int64_t u = 0; u < nk / Gk; u++) {
                uint16_t *ku = kside + (s * max_kunits + u) * 2 * D;
                int64_t kg = (s * (nk / Gk) + u) * D;
                for (int c = 0; c < D; c++) {
                    ku[c] = kscale16[kg + c];
                    ku[D + c] = kzero16[kg + c];
                }
            }
    }
    free(kd);
    free(vd);
    free(kb);
    free(vb);
}

/* The window policy's blocks at G = 32: keys and values of the first nq tokens. */
void oracle_pack_blocks(int B, int H, int64_t nq, int bits, int64_t max_groups,
                        const uint8_t *kcodes, const uint16_t *kzero16,
                        const uint16_t *kscale16,
                        const uint8_t *vcodes, const uint16_t *vzero16,
                        const uint16_t *vscale16, uint8_t *out)
{
    oracle_pack_blocks_kv(B, H, 32, nq, nq, bits, max_groups, 0, kcodes, kzero16, kscale16,
                          vcodes, vzero16, vscale16, out, NULL);
}

/* Outlier records of the packed cache, one per 32-token key group (G = 32):
   256 bytes = uint16 channel[3] (ascending; 0xFFFF when unused), 10 bytes of
   zeros, then fp16 values [3][32] at byte 16 + 64 o (0 when unused).  out
   [B*H][max_groups][256]; groups past nk / 32 are left as they are. */
void oracle_pack_outlier_records(int B, int H, int64_t nk, int n_out, int64_t max_groups,
                                 const int32_t *kout_idx, const uint16_t *kout_val,
                                 uint8_t *out)
{
    const int T = 32;
    for (int64_t s = 0; s < (int64_t)B * H; s++)
        for (int64_t j = 0; j < nk / T; j++) {
            uint8_t *rec = out + (s * max_groups + j) * 256;
            uint16_t *idx = (uint16_t *)rec;
            uint16_t *val = (uint16_t *)(rec + 16);
            memset(rec, 0, 256);
            for (int o = 0; o < 3; o++) idx[o] = 0xFFFF;
            for (int o = 0; o < n_out; o++) {
                int64_t g = s * (nk / T) + j;
                idx[o] = (uint16_t)kout_idx[g * n_out + o];
                for (int i = 0; i < T; i++) val[o * T + i] = kout_val[(g * n_out + o) * T + i];
            }
        }
}

/* Position of one code in the packed area (exported for the layout tests). */
void oracle_code_position(int bits, int is_v, int token, int channel,
                          int64_t *dword, int *bit)
{
    code_position(bits, is_v, token, channel, dword, bit);
}

/* ------------------------------------------------------------------------ */
/* Notebook-style fake quantization of a 2-D float32 array ([NB]             */
/* quantize_grouped): groups of `group` consecutive elements along `axis`    */
/* (0: down a column, as for keys; 1: along a row, as for values); the       */
/* length along `axis` must be a multiple of `group` (no partial groups).    */
/* mode 0: reconstruct with the stored fp16 pair (this cache's view);        */
/* mode 1: reconstruct with the float32 pair, x_min + q * scale ([NB]).      */
/* ------------------------------------------------------------------------ */
void oracle_fake_quant_2d(const float *x, int rows, int cols, int axis,
                          int bits, int group, int mode, float *out)
{
    float *g = (float *)malloc(sizeof(float) * (size_t)group);
    uint8_t *c = (uint8_t *)malloc((size_t)group);
    int len = axis == 0 ? rows : cols;      /* along the group axis */
    int other = axis == 0 ? cols : rows;
    for (int o = 0; o < other; o++)
        for (int j = 0; j < len / group; j++) {
            for (int i = 0; i < group; i++) {
                int r = axis == 0 ? j * group + i : o;
                int cc = axis == 0 ? o : j * group + i;
                g[i] = x[(int64_t)r * cols + cc];
            }
            float mn, s;
            uint16_t z16, s16;
            oracle_group_quant(g, group, bits, c, &mn, &s, &z16, &s16);
            for (int i = 0; i < group; i++) {
                int r = axis == 0 ? j * group + i : o;
                int cc = axis == 0 ? o : j * group + i;
                float xh;
                if (mode == 0) {
                    xh = oracle_dequant_one(c[i], z16, s16);
                } else {
                    float p = (float)c[i] * s;
                    xh = mn + p;
                }
                out[(int64_t)r * cols + cc] = xh;
            }
        }
    free(g);
    free(c);
}

/* Array forms of the fp16 conversions (for the tests). */
void oracle_f16_to_f32_array(const uint16_t *h, float *f, int64_t n)
{
    for (int64_t i = 0; i < n; i++) f[i] = oracle_f16_to_f32(h[i]);
}

void oracle_f32_to_f16_array(const float *f, uint16_t *h, int64_t n)
{
    for (int64_t i = 0; i < n; i++) h[i] = oracle_f32_to_f16(f[i]);
}
