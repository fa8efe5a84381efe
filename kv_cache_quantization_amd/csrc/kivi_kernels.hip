// kivi_kernels.hip -- KIVI hot-path kernels for CDNA4 (gfx950), wave64.
//
// What the kernels compute (pages cited by title and section):
//  * quantize: "KIVI - 2-bit KV cache quantisation" (cookbook notebook),
//    "Asymmetric 2-bit quantiser": per group zero = min, scale =
//    (max - min) / (2^b - 1) with scale 1 for a constant group, code =
//    round((x - zero) / scale) clamped to [0, 2^b - 1].  Keys are grouped
//    per channel over G consecutive tokens, values per token over G
//    consecutive channels ("KIVI", VeloxQuant-MLX docs, "How it works" 1-2).
//  * residual ring + whole-group flush: same docs, items 3-4.
//  * decode attention with dequantization inside the products:
//    "[Paper review] KIVI ... (ICML'24)", 1.3 decoding step and 3.2
//    system-level implementation (fused dequantize + matmul).
//
// Packed block of one (stream, token group) -- see also include/kivi.h:
//   [K codes | V codes | K scale[128] | K zero[128] | V scale[4][32] | V zero[4][32]]
// Code area order (b bits per code, 64 lanes, 2b dwords per lane): lane l's
// dword w is dword (w/4)*256 + 4*l + (w%4).  Within a dword, slot i
// (0 <= i < 16/b) of half h sits at bit 16h + b*i and feeds matrix-core
// operand o = w*(4/b) + i/4 at position kk = 2*(i%4) + h:
//   keys:   token = 16*(o/4) + l%16,   channel = 32*(o%4) + 8*(l/16) + kk
//   values: channel = 16*o + l%16,     token = 4*(l/16) + kk%4 + 16*(kk/4)
// so that  ((dword >> (b*(4*(o%(4/b)) + m))) & mask2)  is, as two fp16 bit
// patterns, the pair (kk = 2m, 2m+1) of operand o -- one shift and one AND
// per two codes, and every lane's 16 bytes are exactly its own operands.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>
#include "kivi_internal.h"

namespace kivi {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int D = kHeadDim;
constexpr int G = kGroup;

// ===========================================================================
// Quantization: one wavefront per (stream, token group, K-or-V).
// ===========================================================================

// Row t of a stream: from the ring if it was appended earlier, else from the
// new chunk.
template <typename T>
__device__ __forceinline__ const T *source_row(const QuantizeArgs &a, const void *ring,
                                               const void *in, int64_t stream, int64_t t) {
    if (t < a.n_old)
        return (const T *)ring + (stream * a.ring_cap + t % a.ring_cap) * D;
    return (const T *)in + (stream * a.n_new + (t - a.n_old)) * D;
}

__device__ __forceinline__ void load8(const _Float16 *p, float *x) {
    uint4 u = *(const uint4 *)p;
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; e++) {
        h2 v = __builtin_bit_cast(h2, w[e]);
        x[2 * e] = (float)v[0];
        x[2 * e + 1] = (float)v[1];
    }
}

__device__ __forceinline__ void load8(const float *p, float *x) {
    float4 u0 = *(const float4 *)p, u1 = *(const float4 *)(p + 4);
    x[0] = u0.x; x[1] = u0.y; x[2] = u0.z; x[3] = u0.w;
    x[4] = u1.x; x[5] = u1.y; x[6] = u1.z; x[7] = u1.w;
}

__device__ __forceinline__ float xmin(float v, int m) { return fminf(v, __shfl_xor(v, m)); }
__device__ __forceinline__ float xmax(float v, int m) { return fmaxf(v, __shfl_xor(v, m)); }

// Code of one element: IEEE float32 subtract and divide, round half to even,
// clamp -- exactly the quantiser's formula, no reassociation.
__device__ __forceinline__ uint32_t quant_code(float x, float mn, float s, float L) {
    float d = x - mn;
    float t = d / s;
    float c = __builtin_rintf(t);
    c = fminf(fmaxf(c, 0.0f), L);
    return (uint32_t)c;
}

__device__ __forceinline__ void group_params(float mn, float mx, float L, float &mn_out,
                                             float &s_out) {
    if (mn == 0.0f) mn = 0.0f;      // a zero minimum is +0 whatever the sign
    float s = (mx - mn) / L;
    if (s == 0.0f) s = 1.0f;        // constant group
    mn_out = mn;
    s_out = s;
}

constexpr int kLdsRow = 136;        // 128 code bytes + 8 pad (fewer bank conflicts)

template <int BITS, typename T>
__global__ __launch_bounds__(64) void quantize_kernel(QuantizeArgs a) {
    __shared__ uint8_t codes_lds[G * kLdsRow];
    const int l = threadIdx.x;
    const int64_t ngr = a.group_end - a.group_begin;
    const int64_t task = blockIdx.x;
    const int is_v = (int)(task & 1);
    const int64_t rest = task >> 1;
    const int64_t stream = rest / ngr;
    const int64_t g = a.group_begin + rest % ngr;
    const float L = (float)((1 << BITS) - 1);

    // Load the 32 x 128 tile: load i covers rows 4i..4i+3; lane l holds row
    // 4i + l/16, channels 8*(l%16) .. +7.
    const void *ring = is_v ? a.ring_v : a.ring_k;
    const void *in = is_v ? a.in_v : a.in_k;
    const int rsub = l >> 4;
    const int c0 = 8 * (l & 15);
    float x[8][8];
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const T *row = source_row<T>(a, ring, in, stream, g * G + 4 * i + rsub);
        load8(row + c0, x[i]);
    }

    uint8_t *blk = a.blocks + (stream * a.max_groups + g) * a.block_bytes;
    const int cbytes = BITS * G * D / 8;
    _Float16 *side = (_Float16 *)(blk + 2 * cbytes);   // kscale, kzero, vscale, vzero

    uint32_t code8[8][2];   // per row i: 8 codes as bytes (two dwords)
    if (!is_v) {
        // keys: group = one channel over the 32 rows
        float mn[8], s[8];
#pragma unroll
        for (int e = 0; e < 8; e++) {
            float lo = x[0][e], hi = x[0][e];
#pragma unroll
            for (int i = 1; i < 8; i++) { lo = fminf(lo, x[i][e]); hi = fmaxf(hi, x[i][e]); }
            lo = xmin(xmin(lo, 16), 32);
            hi = xmax(xmax(hi, 16), 32);
            group_params(lo, hi, L, mn[e], s[e]);
        }
        if (l < 16) {
#pragma unroll
            for (int e = 0; e < 8; e++) {
                side[c0 + e] = (_Float16)s[e];
                side[D + c0 + e] = (_Float16)mn[e];
            }
        }
#pragma unroll
        for (int i = 0; i < 8; i++) {
            uint32_t lo = 0, hi = 0;
#pragma unroll
            for (int e = 0; e < 4; e++) lo |= quant_code(x[i][e], mn[e], s[e], L) << (8 * e);
#pragma unroll
            for (int e = 0; e < 4; e++) hi |= quant_code(x[i][4 + e], mn[4 + e], s[4 + e], L) << (8 * e);
            code8[i][0] = lo;
            code8[i][1] = hi;
        }
    } else {
        // values: group = one row over 32 channels (4 lanes of a quad)
        const int cg = (l & 15) >> 2;
#pragma unroll
        for (int i = 0; i < 8; i++) {
            float lo = x[i][0], hi = x[i][0];
#pragma unroll
            for (int e = 1; e < 8; e++) { lo = fminf(lo, x[i][e]); hi = fmaxf(hi, x[i][e]); }
            lo = xmin(xmin(lo, 1), 2);
            hi = xmax(xmax(hi, 1), 2);
            float mn, s;
            group_params(lo, hi, L, mn, s);
            if ((l & 3) == 0) {
                const int r = 4 * i + rsub;
                side[2 * D + cg * G + r] = (_Float16)s;
                side[3 * D + cg * G + r] = (_Float16)mn;
            }
            uint32_t c_lo = 0, c_hi = 0;
#pragma unroll
            for (int e = 0; e < 4; e++) c_lo |= quant_code(x[i][e], mn, s, L) << (8 * e);
#pragma unroll
            for (int e = 0; e < 4; e++) c_hi |= quant_code(x[i][4 + e], mn, s, L) << (8 * e);
            code8[i][0] = c_lo;
            code8[i][1] = c_hi;
        }
    }

    // Redistribute codes (one byte each) through LDS into the packed order.
#pragma unroll
    for (int i = 0; i < 8; i++) {
        uint2 v = {code8[i][0], code8[i][1]};
        *(uint2 *)&codes_lds[(4 * i + rsub) * kLdsRow + c0] = v;
    }
    __syncthreads();

    constexpr int DPL = 2 * BITS;          // dwords per lane
    constexpr int OPD = 4 / BITS;          // operands per dword
    uint32_t outw[DPL];
#pragma unroll
    for (int w = 0; w < DPL; w++) outw[w] = 0;
#pragma unroll
    for (int o = 0; o < 8; o++) {
        uint32_t cb[8];
        if (!is_v) {
            const int tok = 16 * (o >> 2) + (l & 15);
            const int ch = 32 * (o & 3) + 8 * (l >> 4);
            uint2 v = *(const uint2 *)&codes_lds[tok * kLdsRow + ch];
#pragma unroll
            for (int kk = 0; kk < 4; kk++) {
                cb[kk] = (v.x >> (8 * kk)) & 0xFF;
                cb[4 + kk] = (v.y >> (8 * kk)) & 0xFF;
            }
        } else {
            const int ch = 16 * o + (l & 15);
#pragma unroll
            for (int kk = 0; kk < 8; kk++) {
                const int tok = 4 * (l >> 4) + (kk & 3) + 16 * (kk >> 2);
                cb[kk] = codes_lds[tok * kLdsRow + ch];
            }
        }
        const int w = o / OPD;
        const int base = BITS * 4 * (o % OPD);
#pragma unroll
        for (int kk = 0; kk < 8; kk++)
            outw[w] |= cb[kk] << (16 * (kk & 1) + base + BITS * (kk >> 1));
    }
    uint32_t *dst = (uint32_t *)(blk + (is_v ? cbytes : 0));
#pragma unroll
    for (int w4 = 0; w4 < DPL / 4; w4++) {
        uint4 v = {outw[4 * w4], outw[4 * w4 + 1], outw[4 * w4 + 2], outw[4 * w4 + 3]};
        *(uint4 *)&dst[w4 * 256 + 4 * l] = v;
    }
}

// ===========================================================================
// Residual ring append: copy rows [tok_begin, tok_end) of the chunk into
// ring slot t % ring_cap.  16 bytes per thread.
// ===========================================================================
__global__ __launch_bounds__(256) void ring_append_kernel(RingArgs a) {
    const int64_t row_vec = (int64_t)D * a.esize / 16;
    const int64_t ntok = a.tok_end - a.tok_begin;
    const int64_t per_tensor = (int64_t)a.streams * ntok * row_vec;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < 2 * per_tensor;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int which = idx >= per_tensor;
        int64_t r = idx - which * per_tensor;
        const int64_t v = r % row_vec;
        r /= row_vec;
        const int64_t t = a.tok_begin + r % ntok;
        const int64_t stream = r / ntok;
        const uint4 *src = (const uint4 *)((const uint8_t *)(which ? a.in_v : a.in_k) +
                                           (stream * a.n_new + (t - a.n_old)) * D * a.esize);
        uint4 *dst = (uint4 *)((uint8_t *)(which ? a.ring_v : a.ring_k) +
                               (stream * a.ring_cap + t % a.ring_cap) * D * a.esize);
        dst[v] = src[v];
    }
}

// ===========================================================================
// Decode attention.
//
// Work items (one wavefront = one workgroup each): first one "tail" item per
// stream over the full-precision residual, then `splits` items per stream
// over whole groups of the quantized prefix.  Each writes an unnormalized
// partial (m, l, o) in the log2 domain; decode_combine_kernel merges them.
//
// Quantized groups use the matrix cores (v_mfma_f32_16x16x32_f16).  With
// GQ query heads per KV head, column j of every B operand belongs to query
// head j % GQ, so the scores come out replicated across columns and each
// lane already holds what it needs for the value product:
//   scores  S^T[token][j]   = sum_c code_K[token][c] * (q[j%GQ][c] * kscale[c])
//                             + sum_c q[j%GQ][c] * kzero[c]
//   values  O^T[chan][j]    = sum_t code_V[t][chan] * (p[t][j%GQ] * vscale[t][cg(j)])
//                             + sum_t p[t][j%GQ] * vzero[t][cg(j)]
// where cg(j) = j / GQ picks the value channel group whose scale the column
// carries; only the M-tiles of that group are kept from each column.
// Codes enter the matrix core as fp16 subnormal bit patterns (value
// code * 2^-24, exact), so unpacking is a shift and an AND; the 2^24 is
// folded into the softmax scale and the final store.
//
// Memory pipeline: a lane's 16 bytes of K codes and 16 bytes of V codes are
// exactly its own operands, so they go straight to registers; the 1 KiB of
// zero/scale data of a group is loaded coalesced (16 bytes per lane) and
// staged through 1 KiB of LDS so every lane can read the entries of its own
// channels / tokens.  The next group's loads are issued before the current
// group is computed.
// ===========================================================================

// Reductions over the four 16-lane rows (lanes j, j+16, j+32, j+48) with
// gfx950's v_permlane32_swap (exchange the two 32-lane halves) and
// v_permlane16_swap (exchange odd and even rows): vector-ALU moves, no LDS
// round trip.  s_nop 1 covers the VALU-write -> permlane-read hazard.
__device__ __forceinline__ void swap_halves(float &a, float &b) {
    asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void swap_rows(float &a, float &b) {
    asm("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ float xsum_rows(float v) {
    float a = v, b = v;
    swap_halves(a, b);
    float c = a + b, d = c;
    swap_rows(c, d);
    return c + d;
}
__device__ __forceinline__ float xmax_rows(float v) {
    float a = v, b = v;
    swap_halves(a, b);
    float c = fmaxf(a, b), d = c;
    swap_rows(c, d);
    return fmaxf(c, d);
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) v += __shfl_xor(v, m);
    return v;
}

// Matrix-core operand o from a lane's code dwords.  Pair m of the operand
// (positions kk = 2m, 2m+1) is taken with one AND, in place: at 2 bits the
// codes of pair m sit at bits 2m and 16 + 2m of the (for odd o, 8-bit
// shifted) dword, so the fp16 subnormals read code * 4^m * 2^-24; at 4 bits
// pairs m = 0,1 sit at bits 4m, 16 + 4m and pairs 2,3 at the same bits of
// the dword shifted by 8, reading code * 16^(m&1) * 2^-24.  The factor
// 2^kScaleLog2<BITS>(m) is divided out of the other operand.
template <int BITS>
__device__ __forceinline__ constexpr int kScaleLog2(int m) {
    return BITS == 2 ? 2 * m : BITS == 4 ? 4 * (m & 1) : 0;
}

template <int BITS>
__device__ __forceinline__ h8 unpack_operand(const uint32_t *w, int o) {
    constexpr uint32_t M1 = (1u << BITS) - 1u;
    constexpr uint32_t MASK = M1 | (M1 << 16);
    uint32_t r[4];
    if (BITS == 2) {
        const uint32_t x = (o & 1) ? (w[o >> 1] >> 8) : w[o >> 1];
#pragma unroll
        for (int m = 0; m < 4; m++) r[m] = x & (MASK << (2 * m));
    } else {
        const uint32_t x = w[o], y = x >> 8;
#pragma unroll
        for (int m = 0; m < 4; m++) r[m] = (m < 2 ? x : y) & (MASK << (4 * (m & 1)));
    }
    uint4 u = {r[0], r[1], r[2], r[3]};
    return __builtin_bit_cast(h8, u);
}

__device__ __forceinline__ h8 pack_h8(const h2 *v) {
    h8 r;
#pragma unroll
    for (int m = 0; m < 4; m++) { r[2 * m] = v[m][0]; r[2 * m + 1] = v[m][1]; }
    return r;
}

__device__ __forceinline__ void split4(u32x4 u, h2 *v) {
    v[0] = __builtin_bit_cast(h2, u.x);
    v[1] = __builtin_bit_cast(h2, u.y);
    v[2] = __builtin_bit_cast(h2, u.z);
    v[3] = __builtin_bit_cast(h2, u.w);
}

__device__ __forceinline__ void split4(uint4 u, h2 *v) {
    v[0] = __builtin_bit_cast(h2, u.x);
    v[1] = __builtin_bit_cast(h2, u.y);
    v[2] = __builtin_bit_cast(h2, u.z);
    v[3] = __builtin_bit_cast(h2, u.w);
}

__device__ __forceinline__ float load_q(const DecodeArgs &a, int64_t idx) {
    return a.q_is_f32 ? ((const float *)a.q)[idx] : (float)((const _Float16 *)a.q)[idx];
}

// q of query head hq as fp16 pairs in B-operand order: slice s, pair m ->
// channels 32s + 8*Gl + 2m, +1 (one 16-byte load per slice for fp16 q).
__device__ __forceinline__ void load_q_operand(const DecodeArgs &a, int64_t qrow, int Gl,
                                               h2 (&qB)[4][4]) {
    if (a.q_is_f32) {
        const float *q = (const float *)a.q + qrow + 8 * Gl;
#pragma unroll
        for (int s = 0; s < 4; s++) {
            const float4 x0 = *(const float4 *)(q + 32 * s);
            const float4 x1 = *(const float4 *)(q + 32 * s + 4);
            qB[s][0] = (h2){(_Float16)x0.x, (_Float16)x0.y};
            qB[s][1] = (h2){(_Float16)x0.z, (_Float16)x0.w};
            qB[s][2] = (h2){(_Float16)x1.x, (_Float16)x1.y};
            qB[s][3] = (h2){(_Float16)x1.z, (_Float16)x1.w};
        }
    } else {
        const _Float16 *q = (const _Float16 *)a.q + qrow + 8 * Gl;
#pragma unroll
        for (int s = 0; s < 4; s++) split4(*(const uint4 *)(q + 32 * s), qB[s]);
    }
}

// Online-softmax step over the 8 scores a lane holds (two 16-token tiles),
// shared by the quantized and the residual paths.  Returns p as fp16 pairs
// in value-operand order, pair m pre-divided by 2^kScaleLog2<SB>(m) (SB = 0:
// no scaling); l_run accumulates the unscaled sum.  nm[m] caches
// -m_run - kScaleLog2<SB>(m).
template <int SB>
__device__ __forceinline__ void softmax_step(const f4 &S0, const f4 &S1, float cs, float kbl,
                                             float &m_run, float (&nm)[4], float &l_run,
                                             float (&vb)[4], f4 (&accV)[8], h2 (&P)[4]) {
    float mt = fmaxf(fmaxf(fmaxf(S0[0], S0[1]), fmaxf(S0[2], S0[3])),
                     fmaxf(fmaxf(S1[0], S1[1]), fmaxf(S1[2], S1[3])));
    mt = __builtin_fmaf(xmax_rows(mt), cs, kbl);
    const float m_new = fmaxf(m_run, mt);
    if (__any(m_new > m_run)) {
        const float al = __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
        for (int o = 0; o < 8; o++) accV[o] *= al;
        l_run *= al;
#pragma unroll
        for (int m = 0; m < 4; m++) {
            vb[m] *= al;
            nm[m] = -m_new - (float)kScaleLog2<SB>(m);
        }
        m_run = m_new;
    }
    float nk[4];
#pragma unroll
    for (int m = 0; m < 4; m++) nk[m] = nm[m] + kbl;
    float p[8];
#pragma unroll
    for (int e = 0; e < 4; e++) {
        p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(S0[e], cs, nk[e >> 1]));
        p[4 + e] = __builtin_amdgcn_exp2f(__builtin_fmaf(S1[e], cs, nk[2 + (e >> 1)]));
    }
#pragma unroll
    for (int m = 0; m < 4; m++) {
        const _Float16 up = (_Float16)(float)(1 << kScaleLog2<SB>(m));
        const h2 w = {up, up};
        P[m][0] = (_Float16)p[2 * m];
        P[m][1] = (_Float16)p[2 * m + 1];
        l_run = __builtin_amdgcn_fdot2(P[m], w, l_run, false);
    }
}

// Store a partial: lanes whose column carries value channel group cg write
// the two M-tiles of that group; one lane per head writes (m, l).
template <int GQ>
__device__ __forceinline__ void store_partial(const DecodeArgs &a, int64_t pi, int l,
                                              const f4 (&accV)[8], float scale, float bias,
                                              float m_run, float l_tot) {
    const int j = l & 15, Gl = l >> 4;
    const int cg = (j / GQ) & 3;
    if (j < 4 * GQ) {
        // tiles 2cg and 2cg+1, chosen with selects (a lane-dependent array
        // index would push the accumulators to scratch memory)
#pragma unroll
        for (int e = 0; e < 2; e++) {
            const f4 t = cg == 0 ? accV[e] : cg == 1 ? accV[2 + e] : cg == 2 ? accV[4 + e]
                                                                                : accV[6 + e];
            float4 v;
            v.x = __builtin_fmaf(t[0], scale, bias);
            v.y = __builtin_fmaf(t[1], scale, bias);
            v.z = __builtin_fmaf(t[2], scale, bias);
            v.w = __builtin_fmaf(t[3], scale, bias);
            *(float4 *)&a.part_o[pi * D + 16 * (2 * cg + e) + 4 * Gl] = v;
        }
    }
    if (j < GQ && Gl == 0) {
        a.part_ml[2 * pi] = m_run;
        a.part_ml[2 * pi + 1] = l_tot;
    }
}

constexpr float kTwo24 = 16777216.0f;
constexpr float kTwoM24 = 5.9604644775390625e-08f;

// Residual item, fp16 ring: tokens [n_quant, n) in chunks of 32 through the
// same matrix-core products (K rows and q are exact fp16, no scale/zero).
template <int GQ>
__device__ void decode_tail_f16(const DecodeArgs &a, int stream) {
    const int l = threadIdx.x & 63;
    const int j = l & 15, Gl = l >> 4;
    const int h = j % GQ;
    const int b = stream / a.kv_heads, hk = stream % a.kv_heads;
    const int hq = hk * GQ + h;
    const int items = a.splits + 1;
    h2 qB[4][4];
    load_q_operand(a, ((int64_t)b * a.q_heads + hq) * D, Gl, qB);
    const _Float16 *rk = (const _Float16 *)a.ring_k + (int64_t)stream * a.ring_cap * D;
    const _Float16 *rv = (const _Float16 *)a.ring_v + (int64_t)stream * a.ring_cap * D;
    float m_run = -INFINITY, l_run = 0.f;
    float nm[4] = {INFINITY, INFINITY, INFINITY, INFINITY}, vb[4] = {0.f, 0.f, 0.f, 0.f};
    f4 accV[8];
#pragma unroll
    for (int o = 0; o < 8; o++) accV[o] = (f4){0.f, 0.f, 0.f, 0.f};
    for (int64_t base = a.n_quant; base < a.n_tokens; base += G) {
        f4 S[2];
#pragma unroll
        for (int t = 0; t < 2; t++) {
            const int64_t tok = base + 16 * t + (l & 15);
            const bool ok = tok < a.n_tokens;
            const int64_t tc = ok ? tok : a.n_tokens - 1;
            const _Float16 *row = rk + (tc % a.ring_cap) * D + 8 * Gl;
            S[t] = (f4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; s++) {
                uint4 u = *(const uint4 *)(row + 32 * s);
                if (!ok) u = (uint4){0u, 0u, 0u, 0u};
                S[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, u),
                                                             pack_h8(qB[s]), S[t], 0, 0, 0);
            }
            // lane (j, Gl) holds tokens base + 16t + 4Gl + e
#pragma unroll
            for (int e = 0; e < 4; e++)
                if (base + 16 * t + 4 * Gl + e >= a.n_tokens) S[t][e] = -INFINITY;
        }
        h2 P[4];
        softmax_step<0>(S[0], S[1], a.sm_log2, 0.0f, m_run, nm, l_run, vb, accV, P);
        const h8 Bp = pack_h8(P);
#pragma unroll
        for (int o = 0; o < 8; o++) {
            const int c = 16 * o + (l & 15);
            h8 A;
#pragma unroll
            for (int kk = 0; kk < 8; kk++) {
                // unconditional load from a valid slot, then zero past the end
                const int64_t tok = base + 4 * Gl + (kk & 3) + 16 * (kk >> 2);
                const int64_t tc = tok < a.n_tokens ? tok : a.n_tokens - 1;
                const _Float16 x = rv[(tc % a.ring_cap) * D + c];
                A[kk] = tok < a.n_tokens ? x : (_Float16)0.0f;
            }
            accV[o] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, Bp, accV[o], 0, 0, 0);
        }
    }
    const int64_t pi = ((int64_t)b * a.q_heads + hq) * items + a.splits;
    store_partial<GQ>(a, pi, l, accV, 1.0f, 0.0f, m_run, xsum_rows(l_run));
}

// Residual item, fp32 ring: one token per step on the vector ALUs (lane l
// owns channels 2l, 2l+1), online softmax in the log2 domain.
template <int GQ>
__device__ void decode_tail_f32(const DecodeArgs &a, int stream) {
    const int l = threadIdx.x & 63;
    const int b = stream / a.kv_heads, hk = stream % a.kv_heads;
    const int items = a.splits + 1;
    const float *rk = (const float *)a.ring_k;
    const float *rv = (const float *)a.ring_v;
    float q0[GQ], q1[GQ], m[GQ], ls[GQ], a0[GQ], a1[GQ];
#pragma unroll
    for (int h = 0; h < GQ; h++) {
        const int64_t qrow = ((int64_t)b * a.q_heads + hk * GQ + h) * D;
        q0[h] = load_q(a, qrow + 2 * l);
        q1[h] = load_q(a, qrow + 2 * l + 1);
        m[h] = -INFINITY;
        ls[h] = 0.f;
        a0[h] = 0.f;
        a1[h] = 0.f;
    }
    for (int64_t t = a.n_quant; t < a.n_tokens; t++) {
        const int64_t row = ((int64_t)stream * a.ring_cap + t % a.ring_cap) * D + 2 * l;
        const float k0 = rk[row], k1 = rk[row + 1], v0 = rv[row], v1 = rv[row + 1];
#pragma unroll
        for (int h = 0; h < GQ; h++) {
            float s = wave_sum(__builtin_fmaf(q0[h], k0, q1[h] * k1)) * a.sm_log2;
            float mn = fmaxf(m[h], s);
            float al = __builtin_amdgcn_exp2f(m[h] - mn);
            float p = __builtin_amdgcn_exp2f(s - mn);
            ls[h] = __builtin_fmaf(ls[h], al, p);
            a0[h] = __builtin_fmaf(a0[h], al, p * v0);
            a1[h] = __builtin_fmaf(a1[h], al, p * v1);
            m[h] = mn;
        }
    }
#pragma unroll
    for (int h = 0; h < GQ; h++) {
        const int64_t pi = ((int64_t)b * a.q_heads + hk * GQ + h) * items + a.splits;
        float2 ov = {a0[h], a1[h]};
        *(float2 *)&a.part_o[pi * D + 2 * l] = ov;
        if (l == 0) {
            a.part_ml[2 * pi] = m[h];
            a.part_ml[2 * pi + 1] = ls[h];
        }
    }
}

// LDS pipeline of packed blocks.  Each group's block (codes + side data,
// 3 KiB at 2 bits, 5 KiB at 4 bits) is copied verbatim into one of NST LDS
// stages with global_load_lds_dwordx4 (64 lanes x 16 bytes = 1 KiB per
// instruction, straight from HBM into LDS, no registers), NST - 1 groups
// ahead of the one being computed.  The copies are issued and awaited with
// inline assembly: the compiler's own wait insertion would otherwise wait for
// every outstanding copy before each LDS read.
template <int BITS>
struct Pipe {
    static constexpr int CB = BITS * G * D / 8;         // code bytes per tensor
    static constexpr int BB = 2 * CB + 4 * D * 2;       // block bytes
    static constexpr int DPG = BB / 1024;               // 1 KiB copies per group
    static constexpr int NST = BITS == 2 ? 3 : 2;       // stages
};

__device__ __forceinline__ void dma_1k(const uint8_t *src_lane, uint32_t lds_dst) {
    // LDS destination: M0 + 16 * lane
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(src_lane), "s"(lds_dst)
                 : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vm() {
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

template <int BITS>
__device__ __forceinline__ void issue_group(const uint8_t *blk, uint32_t stage, int l) {
    asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");   // prior reads of the stage done
#pragma unroll
    for (int c = 0; c < Pipe<BITS>::DPG; c++)
        dma_1k(blk + c * 1024 + 16 * l, __builtin_amdgcn_readfirstlane(stage + c * 1024));
}

// Wait until at most `r` groups (issued after the one needed) are in flight.
template <int BITS>
__device__ __forceinline__ void wait_groups_after(int r) {
    constexpr int P = Pipe<BITS>::DPG;
    if (r >= 3) wait_vm<3 * P>();
    else if (r == 2) wait_vm<2 * P>();
    else if (r == 1) wait_vm<P>();
    else wait_vm<0>();
}

template <int BITS, int GQ>
__device__ void decode_split(const DecodeArgs &a, int stream, int sp, uint8_t *pipe,
                             uint4 *q_lds) {
    using PP = Pipe<BITS>;
    constexpr int DPL = 2 * BITS;              // code dwords per lane
    const int l = threadIdx.x & 63;
    const int j = l & 15, Gl = l >> 4;
    const int h = j % GQ;
    const int cg = (j / GQ) & 3;
    const int b = stream / a.kv_heads, hk = stream % a.kv_heads;
    const int hq = hk * GQ + h;
    const int items = a.splits + 1;
    const int64_t ng = a.n_quant / G;
    const int64_t g0 = (int64_t)sp * a.groups_per_split;
    const int64_t g1 = g0 + a.groups_per_split < ng ? g0 + a.groups_per_split : ng;

    // q pair m divided by 2^kScaleLog2(m): it meets key codes read in place
    h2 qB[4][4];
    load_q_operand(a, ((int64_t)b * a.q_heads + hq) * D, Gl, qB);
    // Unscaled fp16 q of the GQ heads staged in LDS (16 bytes per lane, head
    // (l/16) % GQ, channels 8*(l%16)..+7): B operand of the key-zero product.
    {
        const int64_t qoff = ((int64_t)b * a.q_heads + hk * GQ + (l >> 4) % GQ) * D + 8 * (l & 15);
        uint4 u;
        if (a.q_is_f32) {
            const float *qf = (const float *)a.q + qoff;
            const float4 x0 = *(const float4 *)qf, x1 = *(const float4 *)(qf + 4);
            h2 t0 = {(_Float16)x0.x, (_Float16)x0.y}, t1 = {(_Float16)x0.z, (_Float16)x0.w};
            h2 t2 = {(_Float16)x1.x, (_Float16)x1.y}, t3 = {(_Float16)x1.z, (_Float16)x1.w};
            u.x = __builtin_bit_cast(uint32_t, t0); u.y = __builtin_bit_cast(uint32_t, t1);
            u.z = __builtin_bit_cast(uint32_t, t2); u.w = __builtin_bit_cast(uint32_t, t3);
        } else {
            u = *(const uint4 *)((const _Float16 *)a.q + qoff);
        }
        q_lds[l] = u;
    }
#pragma unroll
    for (int m = 0; m < 4; m++) {
        const _Float16 dn = (_Float16)(1.0f / (float)(1 << kScaleLog2<BITS>(m)));
        const h2 d2 = {dn, dn};
#pragma unroll
        for (int s = 0; s < 4; s++) qB[s][m] = qB[s][m] * d2;
    }
    const float cs = a.sm_log2 * kTwo24;        // score units -> log2 units

    float m_run = -INFINITY, l_run = 0.f;
    float nm[4] = {INFINITY, INFINITY, INFINITY, INFINITY}, vb[4] = {0.f, 0.f, 0.f, 0.f};
    f4 accV[8];
#pragma unroll
    for (int o = 0; o < 8; o++) accV[o] = (f4){0.f, 0.f, 0.f, 0.f};

    const uint8_t *sblk = a.blocks + (int64_t)stream * a.max_groups * a.block_bytes;
    const uint32_t pbase = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void *)pipe;
    // q must be in registers before the copies start, and the compiler must
    // know it (its wait tracking does not see the inline-assembly copies).
#pragma unroll
    for (int s = 0; s < 4; s++)
#pragma unroll
        for (int m = 0; m < 4; m++) asm volatile("" : : "v"(qB[s][m]));
    wait_vm<0>();
    int64_t issued = g0;
    for (int st = 0; st < PP::NST - 1 && issued < g1; st++, issued++)
        issue_group<BITS>(sblk + issued * PP::BB, pbase + (uint32_t)((issued - g0) % PP::NST) * PP::BB, l);

    for (int64_t g = g0; g < g1; g++) {
        if (issued < g1) {
            issue_group<BITS>(sblk + issued * PP::BB,
                              pbase + (uint32_t)((issued - g0) % PP::NST) * PP::BB, l);
            issued++;
        }
        wait_groups_after<BITS>((int)(issued - 1 - g));
        const uint8_t *stg = pipe + ((g - g0) % PP::NST) * PP::BB;
        const uint4 *side = (const uint4 *)(stg + 2 * PP::CB);
        uint32_t kc[DPL], vc[DPL];
#pragma unroll
        for (int w4 = 0; w4 < BITS / 2; w4++) {
            const uint4 u = *(const uint4 *)(stg + w4 * 1024 + 16 * l);
            const uint4 v = *(const uint4 *)(stg + PP::CB + w4 * 1024 + 16 * l);
            kc[4 * w4] = u.x; kc[4 * w4 + 1] = u.y; kc[4 * w4 + 2] = u.z; kc[4 * w4 + 3] = u.w;
            vc[4 * w4] = v.x; vc[4 * w4 + 1] = v.y; vc[4 * w4 + 2] = v.z; vc[4 * w4 + 3] = v.w;
        }
        // side data as 16-byte units: kscale 0..15, kzero 16..31, vscale
        // 32..47, vzero 48..63 (channel c at byte 2c of its array, value token
        // t of channel group cg at byte 2(32cg + t)).
        // key-zero bias sum_c q[c] kzero[c] on the matrix core: A = kzero of
        // the lane's channels (the same for every token row), B = unscaled q;
        // every row of Sk then holds the bias of its column's head.
        f4 Sk = (f4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; s++)
            Sk = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                __builtin_bit_cast(h8, side[16 + 4 * s + Gl]),
                __builtin_bit_cast(h8, q_lds[16 * (j % GQ) + 4 * s + Gl]), Sk, 0, 0, 0);
        f4 S0 = (f4){0.f, 0.f, 0.f, 0.f}, S1 = S0;
#pragma unroll
        for (int s = 0; s < 4; s++) {
            // q * kscale carried as an fp16 pair hi + lo, lo = fma(q, kscale,
            // -hi) rounded once: the matrix core sees the product (almost) exactly.
            h2 ks[4], qh[4], ql[4];
            split4(side[4 * s + Gl], ks);
#pragma unroll
            for (int m = 0; m < 4; m++) {
                qh[m] = qB[s][m] * ks[m];
                ql[m] = __builtin_elementwise_fma(qB[s][m], ks[m], -qh[m]);
            }
            const h8 A0 = unpack_operand<BITS>(kc, s), A1 = unpack_operand<BITS>(kc, 4 + s);
            const h8 Bh = pack_h8(qh), Bl = pack_h8(ql);
            S0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A0, Bh, S0, 0, 0, 0);
            S1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A1, Bh, S1, 0, 0, 0);
            S0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A0, Bl, S0, 0, 0, 0);
            S1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A1, Bl, S1, 0, 0, 0);
        }
        h2 P[4];
        softmax_step<BITS>(S0, S1, cs, Sk[0] * a.sm_log2, m_run, nm, l_run, vb, accV, P);
        h2 vs[4], vz[4], ps[4];
        {
            const uint2 *s2 = (const uint2 *)side;
            const uint2 a0 = s2[64 + 8 * cg + Gl], a1 = s2[64 + 8 * cg + Gl + 4];
            const uint2 z0 = s2[96 + 8 * cg + Gl], z1 = s2[96 + 8 * cg + Gl + 4];
            vs[0] = __builtin_bit_cast(h2, a0.x); vs[1] = __builtin_bit_cast(h2, a0.y);
            vs[2] = __builtin_bit_cast(h2, a1.x); vs[3] = __builtin_bit_cast(h2, a1.y);
            vz[0] = __builtin_bit_cast(h2, z0.x); vz[1] = __builtin_bit_cast(h2, z0.y);
            vz[2] = __builtin_bit_cast(h2, z1.x); vz[3] = __builtin_bit_cast(h2, z1.y);
        }
#pragma unroll
        for (int m = 0; m < 4; m++) {
            vb[m] = __builtin_amdgcn_fdot2(P[m], vz[m], vb[m], false);
            ps[m] = P[m] * vs[m];
        }
        const h8 Bv = pack_h8(ps);
#pragma unroll
        for (int o = 0; o < 8; o++)
            accV[o] = __builtin_amdgcn_mfma_f32_16x16x32_f16(unpack_operand<BITS>(vc, o), Bv,
                                                            accV[o], 0, 0, 0);
    }
    float vbt = vb[0];
#pragma unroll
    for (int m = 1; m < 4; m++) vbt = __builtin_fmaf(vb[m], (float)(1 << kScaleLog2<BITS>(m)), vbt);
    const int64_t pi = ((int64_t)b * a.q_heads + hq) * items + sp;
    store_partial<GQ>(a, pi, l, accV, kTwo24, xsum_rows(vbt), m_run, xsum_rows(l_run));
}

template <int BITS, int GQ>
__global__ __launch_bounds__(64) void decode_kernel(DecodeArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t pipe[Pipe<BITS>::NST * Pipe<BITS>::BB];
    __shared__ uint4 q_lds[64];
    const int64_t item = blockIdx.x;
    const int streams = a.batch * a.kv_heads;
    if (item < streams) {
        if (a.ring_is_f32) decode_tail_f32<GQ>(a, (int)item);
        else decode_tail_f16<GQ>(a, (int)item);
        return;
    }
    const int64_t it = item - streams;
    decode_split<BITS, GQ>(a, (int)(it / a.splits), (int)(it % a.splits), pipe, q_lds);
}

// Merge the partials of one (batch, query head).  The split weights
// 2^(m_s - M) are computed once in LDS; each thread then sums one channel.
constexpr int kMaxItems = 4160;

__global__ __launch_bounds__(128) void decode_combine_kernel(DecodeArgs a) {
    __shared__ float w[kMaxItems];
    __shared__ float red[128];
    const int64_t bh = blockIdx.x;
    const int c = threadIdx.x;
    const int items = a.splits + 1;
    const float *ml = a.part_ml + bh * items * 2;
    float M = -INFINITY;
    for (int s = c; s < items; s += 128)
        if (ml[2 * s + 1] > 0.f) M = fmaxf(M, ml[2 * s]);
    red[c] = M;
    __syncthreads();
    for (int off = 64; off > 0; off >>= 1) {
        if (c < off) red[c] = fmaxf(red[c], red[c + off]);
        __syncthreads();
    }
    M = red[0];
    __syncthreads();
    float Lp = 0.f;
    for (int s = c; s < items; s += 128) {
        const float ls = ml[2 * s + 1];
        const float ws = ls > 0.f ? __builtin_amdgcn_exp2f(ml[2 * s] - M) : 0.f;
        w[s] = ws;
        Lp = __builtin_fmaf(ls, ws, Lp);
    }
    red[c] = Lp;
    __syncthreads();
    for (int off = 64; off > 0; off >>= 1) {
        if (c < off) red[c] += red[c + off];
        __syncthreads();
    }
    const float L = red[0];
    const float *po = a.part_o + bh * items * D + c;
    float acc0 = 0.f, acc1 = 0.f, acc2 = 0.f, acc3 = 0.f;
    int s = 0;
    for (; s + 4 <= items; s += 4) {
        acc0 = __builtin_fmaf(po[(int64_t)s * D], w[s], acc0);
        acc1 = __builtin_fmaf(po[(int64_t)(s + 1) * D], w[s + 1], acc1);
        acc2 = __builtin_fmaf(po[(int64_t)(s + 2) * D], w[s + 2], acc2);
        acc3 = __builtin_fmaf(po[(int64_t)(s + 3) * D], w[s + 3], acc3);
    }
    for (; s < items; s++) acc0 = __builtin_fmaf(po[(int64_t)s * D], w[s], acc0);
    a.out[bh * D + c] = ((acc0 + acc1) + (acc2 + acc3)) / L;
}

// ===========================================================================
// Launchers
// ===========================================================================
hipError_t launch_quantize(const QuantizeArgs &a, hipStream_t s) {
    const int64_t tasks = (int64_t)a.streams * (a.group_end - a.group_begin) * 2;
    if (tasks <= 0) return hipSuccess;
    dim3 grid((unsigned)tasks), block(64);
    if (a.bits == 2) {
        if (a.is_f32) hipLaunchKernelGGL((quantize_kernel<2, float>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((quantize_kernel<2, _Float16>), grid, block, 0, s, a);
    } else {
        if (a.is_f32) hipLaunchKernelGGL((quantize_kernel<4, float>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((quantize_kernel<4, _Float16>), grid, block, 0, s, a);
    }
    return hipGetLastError();
}

hipError_t launch_ring_append(const RingArgs &a, hipStream_t s) {
    const int64_t ntok = a.tok_end - a.tok_begin;
    if (ntok <= 0) return hipSuccess;
    const int64_t vecs = 2 * (int64_t)a.streams * ntok * D * a.esize / 16;
    int64_t blocks = (vecs + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(ring_append_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

template <int BITS>
static void launch_decode_bits(const DecodeArgs &a, int gq, dim3 grid, hipStream_t s) {
    if (gq == 4) hipLaunchKernelGGL((decode_kernel<BITS, 4>), grid, dim3(64), 0, s, a);
    else if (gq == 2) hipLaunchKernelGGL((decode_kernel<BITS, 2>), grid, dim3(64), 0, s, a);
    else hipLaunchKernelGGL((decode_kernel<BITS, 1>), grid, dim3(64), 0, s, a);
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t s) {
    const int streams = a.batch * a.kv_heads;
    const int gq = a.q_heads / a.kv_heads;
    const int64_t items = (int64_t)streams * (a.splits + 1);
    if (a.splits + 1 > kMaxItems) return hipErrorInvalidValue;
    dim3 grid((unsigned)items);
    if (a.bits == 2) launch_decode_bits<2>(a, gq, grid, s);
    else launch_decode_bits<4>(a, gq, grid, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(decode_combine_kernel, dim3((unsigned)(a.batch * a.q_heads)), dim3(128), 0,
                       s, a);
    return hipGetLastError();
}

}  // namespace kivi
