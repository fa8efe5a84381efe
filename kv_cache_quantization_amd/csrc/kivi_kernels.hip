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
#include <atomic>
#include "kivi_internal.h"

namespace kivi {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int D = kHeadDim;
constexpr int G = kGroup;

// Four fp16 pairs from 16 loaded bytes.
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

// ===========================================================================
// Cross-lane exchanges with gfx950's v_permlane32_swap (exchange the two
// 32-lane halves of a pair of registers) and v_permlane16_swap (exchange odd
// and even 16-lane rows): vector-ALU moves, no LDS round trip.  s_nop 1
// covers the VALU-write -> permlane-read hazard.
// ===========================================================================
__device__ __forceinline__ void swap_halves(float &a, float &b) {
    asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void swap_rows(float &a, float &b) {
    asm("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}

// ===========================================================================
// Quantization: one wavefront per (stream, token group, K-or-V) task.
//
// Load layout.  Lane l = 16q + c holds the 16-byte channel chunk c
// (channels 8c .. 8c+7) of eight rows of the 32-token tile:
//   keys    row 4j + q                 (j = 0..7)
//   values  row 4q + j%4 + 16*(j/4)    (j = 0..7)
// A key group (one channel over the 32 tokens) then spans lanes c, c+16,
// c+32, c+48 and a value group (one token over 32 channels) the four lanes of
// a quad.  Eight codes that land in the same matrix-core operand (a "unit":
// the 8 channels of one key row, or one value channel over the lane's 8 rows)
// are computed by one lane, so the move into packed order (through LDS) is
// one 16- or 32-bit unit per operand instead of one byte per code.
//
// Codes.  The quantiser's code is round-half-even of RN(d / s) with
// d = RN(x - zero).  The kernel forms t = RN(x * y + RN(-zero * y)) with one
// FMA, y = v_rcp_f32(s) (within 1 ulp of 1/s).  For t <= 16 that is within
// 5 * 2^-20 + 2^-24 * |zero * y| of RN(d / s), so both round to the same
// integer unless t lies within (four times) that distance of a
// half-integer.  A unit with such an element, or with a scale outside
// [2^-126, inf), is recomputed with the IEEE subtract and divide.  The scale itself, RN((max - min) / L), is computed as
// q0 = RN(rng * RN(1/L)) corrected by one FMA residual step, which equals the
// IEEE quotient for L = 3 and L = 15 and every positive finite rng (checked
// exhaustively against IEEE division on the CPU).
// ===========================================================================

// Rows of the tile [t0, t0 + 32) of one stream: row r is token t0 + r, read
// from ring slot (t0 + r) % ring_cap if it was appended earlier (t < n_old),
// else from row t - n_old of the new chunk.  ring_cap >= 32, so the slot
// wraps at most once inside a tile.
template <typename T>
struct RowSource {
    const T *in;        // chunk row of token t0 (may be "negative" if t0 < n_old)
    const T *ring;      // ring base of the stream
    int n_from_ring;    // rows r < n_from_ring come from the ring (0..32)
    int slot0, cap;
    __device__ __forceinline__ RowSource(const QuantizeArgs &a, const void *ring_, const void *in_,
                                         int64_t stream, int64_t t0) {
        const int64_t old = a.n_old - t0;
        n_from_ring = old <= 0 ? 0 : (old >= G ? G : (int)old);
        in = (const T *)in_ + (stream * a.n_new + (t0 - a.n_old)) * D;
        ring = (const T *)ring_ + stream * a.ring_cap * D;
        cap = (int)a.ring_cap;
        slot0 = n_from_ring ? (int)(t0 % a.ring_cap) : 0;
    }
    __device__ __forceinline__ const T *row(int r) const {
        int slot = slot0 + r;
        slot = slot >= cap ? slot - cap : slot;
        return r < n_from_ring ? ring + slot * D : in + r * D;
    }
};

template <bool IS_V>
__device__ __forceinline__ int tile_row(int j, int q) {
    return IS_V ? 4 * q + (j & 3) + 16 * (j >> 2) : 4 * j + q;
}

// The lane's 8 rows x 8 channels, as loaded.
template <typename T> struct Tile;
template <> struct Tile<_Float16> {
    h2 v[8][4];
    __device__ __forceinline__ float at(int j, int e) const { return (float)v[j][e >> 1][e & 1]; }
    // x * y + c with one rounding (v_fma_mix_f32 takes the fp16 x directly)
    __device__ __forceinline__ float fma(int j, int e, float y, float c) const {
        return __builtin_fmaf((float)v[j][e >> 1][e & 1], y, c);
    }
};
template <> struct Tile<float> {
    float v[8][8];
    __device__ __forceinline__ float at(int j, int e) const { return v[j][e]; }
    __device__ __forceinline__ float fma(int j, int e, float y, float c) const {
        return __builtin_fmaf(v[j][e], y, c);
    }
};

// Input rows are read once: non-temporal loads (measured on the long-context
// prefill append: 456 -> 409 us).
typedef unsigned u4nt __attribute__((ext_vector_type(4)));
typedef float f4nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void load_row(Tile<_Float16> &t, int j, const _Float16 *p) {
    const u4nt w = __builtin_nontemporal_load((const u4nt *)p);
    split4((uint4){w.x, w.y, w.z, w.w}, t.v[j]);
}
__device__ __forceinline__ void zero_row(Tile<_Float16> &t, int j) {
#pragma unroll
    for (int e = 0; e < 4; e++) t.v[j][e] = (h2){(_Float16)0.0f, (_Float16)0.0f};
}
__device__ __forceinline__ void zero_row(Tile<float> &t, int j) {
#pragma unroll
    for (int e = 0; e < 8; e++) t.v[j][e] = 0.0f;
}
__device__ __forceinline__ void load_row(Tile<float> &t, int j, const float *p) {
    const f4nt w0 = __builtin_nontemporal_load((const f4nt *)p);
    const f4nt w1 = __builtin_nontemporal_load((const f4nt *)(p + 4));
    const float4 u0 = {w0.x, w0.y, w0.z, w0.w}, u1 = {w1.x, w1.y, w1.z, w1.w};
    t.v[j][0] = u0.x; t.v[j][1] = u0.y; t.v[j][2] = u0.z; t.v[j][3] = u0.w;
    t.v[j][4] = u1.x; t.v[j][5] = u1.y; t.v[j][6] = u1.z; t.v[j][7] = u1.w;
}

// IEEE 754-2019 minimum / maximum (NaN-propagating, -0 < +0): no input
// quieting needed, and gfx950 has three-input packed forms.
__device__ __forceinline__ h2 hmin(h2 a, h2 b) { return __builtin_elementwise_minimum(a, b); }
__device__ __forceinline__ h2 hmax(h2 a, h2 b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float fmin_(float a, float b) { return __builtin_elementwise_minimum(a, b); }
__device__ __forceinline__ float fmax_(float a, float b) { return __builtin_elementwise_maximum(a, b); }

template <typename V>
__device__ __forceinline__ float as_f(V v) { return __builtin_bit_cast(float, v); }
template <typename V>
__device__ __forceinline__ V from_f(float f) { return __builtin_bit_cast(V, f); }

// Min / max over the four lanes c, c+16, c+32, c+48 (all lanes get the result).
template <bool MAX, typename V>
__device__ __forceinline__ V reduce_q(V v) {
    float a = as_f(v), b = a;
    swap_halves(a, b);
    V m = MAX ? __builtin_elementwise_maximum(from_f<V>(a), from_f<V>(b))
              : __builtin_elementwise_minimum(from_f<V>(a), from_f<V>(b));
    float c = as_f(m), d = c;
    swap_rows(c, d);
    return MAX ? __builtin_elementwise_maximum(from_f<V>(c), from_f<V>(d))
               : __builtin_elementwise_minimum(from_f<V>(c), from_f<V>(d));
}

// Min / max over the four lanes of a quad (DPP quad permutations).
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL,
                                                              0xF, 0xF, true));
}
template <bool MAX, typename V>
__device__ __forceinline__ V reduce_quad(V v) {
    V o = from_f<V>(dpp<0xB1>(as_f(v)));          // lanes [1,0,3,2]
    v = MAX ? __builtin_elementwise_maximum(v, o) : __builtin_elementwise_minimum(v, o);
    o = from_f<V>(dpp<0x4E>(as_f(v)));            // lanes [2,3,0,1]
    return MAX ? __builtin_elementwise_maximum(v, o) : __builtin_elementwise_minimum(v, o);
}

// Key groups: the lane's in-lane minimum / maximum of its 8 channels over
// the tile's rows it holds, merged over the G / 32 tiles of a group, then
// reduced over the four lanes c, c+16, c+32, c+48 that hold the other rows.
template <typename T> struct KPart;
template <> struct KPart<_Float16> { h2 mn[4], mx[4]; };
template <> struct KPart<float> { float mn[8], mx[8]; };

__device__ __forceinline__ void kpart_add(const Tile<_Float16> &t, KPart<_Float16> &p, bool first) {
#pragma unroll
    for (int e = 0; e < 4; e++) {
        h2 mn = t.v[0][e], mx = t.v[0][e];
#pragma unroll
        for (int j = 1; j < 8; j++) { mn = hmin(mn, t.v[j][e]); mx = hmax(mx, t.v[j][e]); }
        p.mn[e] = first ? mn : hmin(p.mn[e], mn);
        p.mx[e] = first ? mx : hmax(p.mx[e], mx);
    }
}
__device__ __forceinline__ void kpart_add(const Tile<float> &t, KPart<float> &p, bool first) {
#pragma unroll
    for (int e = 0; e < 8; e++) {
        float mn = t.v[0][e], mx = t.v[0][e];
#pragma unroll
        for (int j = 1; j < 8; j++) { mn = fmin_(mn, t.v[j][e]); mx = fmax_(mx, t.v[j][e]); }
        p.mn[e] = first ? mn : fmin_(p.mn[e], mn);
        p.mx[e] = first ? mx : fmax_(p.mx[e], mx);
    }
}
__device__ __forceinline__ void kpart_finish(KPart<_Float16> &p, float (&lo)[8], float (&hi)[8]) {
#pragma unroll
    for (int e = 0; e < 4; e++) {
        const h2 mn = reduce_q<false>(p.mn[e]), mx = reduce_q<true>(p.mx[e]);
        lo[2 * e] = (float)mn[0]; lo[2 * e + 1] = (float)mn[1];
        hi[2 * e] = (float)mx[0]; hi[2 * e + 1] = (float)mx[1];
    }
}
__device__ __forceinline__ void kpart_finish(KPart<float> &p, float (&lo)[8], float (&hi)[8]) {
#pragma unroll
    for (int e = 0; e < 8; e++) {
        lo[e] = reduce_q<false>(p.mn[e]);
        hi[e] = reduce_q<true>(p.mx[e]);
    }
}

// Value groups of 32 * GT channels: after the quad (32 channels), the lanes
// c ^ 4 (64 channels) and c ^ 8 (128 channels) of the same row.
template <int GT, bool MAX, typename V>
__device__ __forceinline__ V reduce_span(V v) {
#pragma unroll
    for (int x = 4; x < 4 * GT; x <<= 1) {
        const V o = from_f<V>(__shfl_xor(as_f(v), x));
        v = MAX ? __builtin_elementwise_maximum(v, o) : __builtin_elementwise_minimum(v, o);
    }
    return v;
}

// Per-group minimum and maximum for the lane's 8 groups (k = 0..7: channel
// 8c + k for keys, row j = k for values) of one tile.
template <bool IS_V, int GT>
__device__ __forceinline__ void group_minmax(const Tile<_Float16> &t, float (&lo)[8],
                                             float (&hi)[8]) {
    if (!IS_V) {
        KPart<_Float16> p;
        kpart_add(t, p, true);
        kpart_finish(p, lo, hi);
    } else {
#pragma unroll
        for (int jp = 0; jp < 4; jp++) {
            h2 a[2], b[2];
#pragma unroll
            for (int s = 0; s < 2; s++) {
                const h2 *r = t.v[2 * jp + s];
                a[s] = hmin(hmin(r[0], r[1]), hmin(r[2], r[3]));
                b[s] = hmax(hmax(r[0], r[1]), hmax(r[2], r[3]));
            }
            // (row 2jp, row 2jp+1) pairs
            h2 mn = hmin((h2){a[0][0], a[1][0]}, (h2){a[0][1], a[1][1]});
            h2 mx = hmax((h2){b[0][0], b[1][0]}, (h2){b[0][1], b[1][1]});
            mn = reduce_span<GT, false>(reduce_quad<false>(mn));
            mx = reduce_span<GT, true>(reduce_quad<true>(mx));
            lo[2 * jp] = (float)mn[0]; lo[2 * jp + 1] = (float)mn[1];
            hi[2 * jp] = (float)mx[0]; hi[2 * jp + 1] = (float)mx[1];
        }
    }
}

template <bool IS_V, int GT>
__device__ __forceinline__ void group_minmax(const Tile<float> &t, float (&lo)[8],
                                             float (&hi)[8]) {
    if (!IS_V) {
        KPart<float> p;
        kpart_add(t, p, true);
        kpart_finish(p, lo, hi);
    } else {
#pragma unroll
        for (int j = 0; j < 8; j++) {
            float mn = t.v[j][0], mx = t.v[j][0];
#pragma unroll
            for (int e = 1; e < 8; e++) { mn = fmin_(mn, t.v[j][e]); mx = fmax_(mx, t.v[j][e]); }
            lo[j] = reduce_span<GT, false>(reduce_quad<false>(mn));
            hi[j] = reduce_span<GT, true>(reduce_quad<true>(mx));
        }
    }
}

// zero = min (+0 for a zero minimum), scale = RN((max - zero) / L), or 1 for a
// constant group.  RN(x / L) = fma(fma(-q0, L, x), RN(1/L), q0) with
// q0 = RN(x * RN(1/L)) for every positive finite x (L = 3, 15, 255: checked
// on all of them); +inf and NaN ranges take q0, which is then the quotient.
template <int BITS>
__device__ __forceinline__ void group_params(float lo, float hi, float &mn, float &s) {
#pragma clang fp contract(off)
    constexpr float L = (float)((1 << BITS) - 1);
    constexpr float yL = 1.0f / L;
    mn = lo == 0.0f ? 0.0f : lo;
    const float rng = hi - mn;
    const float q0 = rng * yL;
    const float r = __builtin_fmaf(-q0, L, rng);
    float sv = __builtin_fmaf(r, yL, q0);
    sv = sv == sv ? sv : q0;
    s = sv == 0.0f ? 1.0f : sv;
}

// Exact code: IEEE subtract and divide, round half to even, clamp.
__device__ __forceinline__ float exact_code(float x, float mn, float s, float L) {
#pragma clang fp contract(off)
    const float d = x - mn;
    const float t = d / s;
    return fminf(fmaxf(__builtin_rintf(t), 0.0f), L);
}

// Packed position of code kk (0..7) inside its unit: at 2 bits a 16-bit unit
// with even kk in the low byte and odd kk in the high byte, two bits apart;
// at 4 bits a 32-bit unit with even kk in the low half, odd in the high half,
// four bits apart (accumulated as two 16-bit halves); at 8 bits two 32-bit
// dwords p = kk / 4, code kk at bit 8 * ((kk / 2) % 2) + 16 * (kk % 2).
template <int BITS>
__device__ __forceinline__ constexpr float unit_weight(int kk) {
    return BITS == 2 ? (float)(1u << (8 * (kk & 1) + 2 * (kk >> 1)))
                     : (float)(1u << (4 * (kk >> 1)));
}

// Two floats as an fp16 pair (round to nearest even).
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
    return __builtin_bit_cast(uint32_t, (h2){(_Float16)a, (_Float16)b});
}

// 8-bit codes: each unit is two dwords, packed with v_cvt_pk_u8_f32, then
// moved to operand order through LDS (operand o of a lane = its dwords 2o,
// 2o + 1) and stored as 16 dwords per lane.
template <bool IS_V, typename TT>
__device__ __forceinline__ void quantize_pack8(const QuantizeArgs &a, const TT &t,
                                               const float (&mn)[8], const float (&s)[8],
                                               const float (&y)[8], const float (&cz)[8],
                                               float near_tie, bool fast_ok, uint8_t *blk,
                                               uint32_t *tr, uint32_t omask) {
#pragma clang fp contract(off)
    constexpr float L = 255.0f;
    constexpr int DPL = 16;
    constexpr int cbytes = 8 * G * D / 8;
    const int l = threadIdx.x;
    const int q = l >> 4, c = l & 15;
    uint32_t unit[8][2];
#pragma unroll
    for (int u = 0; u < 8; u++) {
        float cd[8];
        float rmax = 0.0f;
#pragma unroll
        for (int kk = 0; kk < 8; kk++) {
            const float tq = IS_V ? t.fma(kk, u, y[kk], cz[kk]) : t.fma(u, kk, y[kk], cz[kk]);
            cd[kk] = __builtin_rintf(tq);
            rmax = fmaxf(rmax, fabsf(tq - cd[kk]));
        }
        if (!(rmax < near_tie) || !fast_ok) {
#pragma unroll
            for (int kk = 0; kk < 8; kk++) {
                const float x = IS_V ? t.at(kk, u) : t.at(u, kk);
                cd[kk] = exact_code(x, mn[kk], s[kk], L);
            }
        }
        if (!IS_V) {
#pragma unroll
            for (int kk = 0; kk < 8; kk++)          // key channels kept in fp16
                if ((omask >> kk) & 1u) cd[kk] = 0.0f;
        }
#pragma unroll
        for (int p = 0; p < 2; p++) {
            uint32_t wv = 0;
            wv = __builtin_amdgcn_cvt_pk_u8_f32(cd[4 * p], 0, wv);
            wv = __builtin_amdgcn_cvt_pk_u8_f32(cd[4 * p + 2], 1, wv);
            wv = __builtin_amdgcn_cvt_pk_u8_f32(cd[4 * p + 1], 2, wv);
            wv = __builtin_amdgcn_cvt_pk_u8_f32(cd[4 * p + 3], 3, wv);
            unit[u][p] = wv;
        }
    }
    if (!IS_V) {
        // key unit (row 4*jj + q (+16 for the second tile), chunk c) -> lane
        // 4*jj + q + 16*(c%4), operand 4*tile + c/4
#pragma unroll
        for (int jj = 0; jj < 4; jj++) {
            const int L_ = 4 * jj + q + 16 * (c & 3);
#pragma unroll
            for (int r = 0; r < 2; r++) {
                const int o = 4 * r + (c >> 2);
                *(uint2 *)&tr[L_ * DPL + 2 * o] = (uint2){unit[jj + 4 * r][0], unit[jj + 4 * r][1]};
            }
        }
    } else {
        // value unit (channel 8c + e over the lane's rows) -> lane
        // 8*(c%2) + e + 16q, operand c/2
        const int o = c >> 1;
#pragma unroll
        for (int e = 0; e < 8; e++) {
            const int L_ = 8 * (c & 1) + e + 16 * q;
            *(uint2 *)&tr[L_ * DPL + 2 * o] = (uint2){unit[e][0], unit[e][1]};
        }
    }
    __syncthreads();
    uint32_t *dst = (uint32_t *)(blk + (IS_V ? cbytes : 0));
#pragma unroll
    for (int w4 = 0; w4 < DPL / 4; w4++)
        *(uint4 *)&dst[w4 * 256 + 4 * l] = *(const uint4 *)&tr[l * DPL + 4 * w4];
}

// The lane's 8 rows x 8 channels of block g of a stream.
template <bool IS_V, bool RING, typename T>
__device__ __forceinline__ void load_tile(const QuantizeArgs &a, int64_t stream, int64_t g,
                                          Tile<T> &t) {
    const int l = threadIdx.x;
    const int q = l >> 4, c = l & 15;
    const RowSource<T> src(a, IS_V ? a.ring_v : a.ring_k, IS_V ? a.in_v : a.in_k, stream, g * G);
    if (!RING) {
        const T *base = src.in + 8 * c;
#pragma unroll
        for (int j = 0; j < 8; j++) load_row(t, j, base + tile_row<IS_V>(j, q) * D);
    } else {
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const int r = tile_row<IS_V>(j, q);
            // value rows at or past v_limit are not quantized (they need
            // not exist yet): zeros in, codes 0 out
            if (IS_V && g * G + r >= a.v_limit) zero_row(t, j);
            else load_row(t, j, src.row(r) + 8 * c);
        }
    }
}

// One task: a key group (GT consecutive blocks starting at block g0: the
// statistics span all of them, and each block is then coded and stored with
// the group's zero / scale), or the values of block g0 (groups of 32 * GT
// channels per token).
// Outlier-aware keys (OUT): a 64-bit key per channel orders channels by the
// group's max |K| (its fp32 bits, monotone for non-negative floats), ties to
// the lower channel; +1 keeps every key above the 0 of "no candidate".
__device__ __forceinline__ uint64_t outlier_key(float lo, float hi, int ch) {
    const float sc = fmaxf(fabsf(lo), fabsf(hi));
    return (((uint64_t)__builtin_bit_cast(uint32_t, sc) << 8) | (uint32_t)(127 - ch)) + 1u;
}
__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
    const uint32_t lo = __shfl_xor((int)(uint32_t)v, m), hi = __shfl_xor((int)(uint32_t)(v >> 32), m);
    return ((uint64_t)hi << 32) | lo;
}

template <int BITS, bool IS_V, bool RING, typename T, int GT, bool OUT = false, bool KSEG = false>
__device__ __forceinline__ void quantize_task(const QuantizeArgs &a, int64_t stream, int64_t g0,
                                              uint32_t *tr) {
#pragma clang fp contract(off)
    constexpr float L = (float)((1 << BITS) - 1);
    const int l = threadIdx.x;
    const int q = l >> 4, c = l & 15;

    Tile<T> t;
    float lo[8], hi[8];
    if constexpr (!IS_V && KSEG) {
        // segment policy: one block, with the minimum / maximum of its
        // segment's channels 8c .. 8c+7
        load_tile<IS_V, RING>(a, stream, g0, t);
        const float *st = a.seg_stats + stream * 256 + 8 * c;
        const float4 l0 = *(const float4 *)st, l1 = *(const float4 *)(st + 4);
        const float4 h0 = *(const float4 *)(st + 128), h1 = *(const float4 *)(st + 132);
        lo[0] = l0.x; lo[1] = l0.y; lo[2] = l0.z; lo[3] = l0.w;
        lo[4] = l1.x; lo[5] = l1.y; lo[6] = l1.z; lo[7] = l1.w;
        hi[0] = h0.x; hi[1] = h0.y; hi[2] = h0.z; hi[3] = h0.w;
        hi[4] = h1.x; hi[5] = h1.y; hi[6] = h1.z; hi[7] = h1.w;
    } else if constexpr (!IS_V && GT > 1) {
        // the last block stays in registers for the first store below
        KPart<T> part;
#pragma unroll 1
        for (int tt = 0; tt < GT; tt++) {
            load_tile<IS_V, RING>(a, stream, g0 + tt, t);
            kpart_add(t, part, tt == 0);
        }
        kpart_finish(part, lo, hi);
    } else {
        load_tile<IS_V, RING>(a, stream, g0, t);
        group_minmax<IS_V, GT>(t, lo, hi);
    }
    // outlier-aware keys: the a.n_out channels with the largest max |K| of
    // the group (bit k of omask: channel 8c + k), in ascending order in och
    uint32_t omask = 0;
    int och[kMaxKeyOutliers] = {0xFFFF, 0xFFFF, 0xFFFF};
    if constexpr (OUT && !IS_V) {
        uint64_t key[8];
#pragma unroll
        for (int k = 0; k < 8; k++) key[k] = outlier_key(lo[k], hi[k], 8 * c + k);
#pragma unroll
        for (int o = 0; o < kMaxKeyOutliers; o++) {
            if (o < a.n_out) {                  // (unrolled: och stays in registers)
                uint64_t best = 0;
#pragma unroll
                for (int k = 0; k < 8; k++)
                    if (!((omask >> k) & 1u) && key[k] > best) best = key[k];
                // over the 16 channel chunks of a row (the four rows agree)
#pragma unroll
                for (int x = 1; x < 16; x <<= 1) {
                    const uint64_t other = shfl_xor_u64(best, x);
                    best = other > best ? other : best;
                }
                const int ch = 127 - (int)((best - 1u) & 0xFFu);
                och[o] = ch;
                if ((ch >> 3) == c) omask |= 1u << (ch & 7);
            }
        }
        // ascending channel order (at most three)
        if (och[1] < och[0]) { const int x = och[0]; och[0] = och[1]; och[1] = x; }
        if (och[2] < och[1]) { const int x = och[1]; och[1] = och[2]; och[2] = x; }
        if (och[1] < och[0]) { const int x = och[0]; och[0] = och[1]; och[1] = x; }
    }
    float mn[8], s[8], y[8], cz[8];
    float smin = INFINITY, smax = 0.0f, czmax = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; k++) {
        group_params<BITS>(lo[k], hi[k], mn[k], s[k]);
        y[k] = __builtin_amdgcn_rcpf(s[k]);
        cz[k] = -mn[k] * y[k];
        smin = fminf(smin, s[k]);
        smax = fmaxf(smax, s[k]);
        czmax = fmaxf(czmax, fabsf(cz[k]));
    }
    // Scales outside [2^-126, inf) and NaN (fails both) take the exact path.
    const bool fast_ok = smin >= 0x1p-126f && smax < INFINITY;
    // t = RN(x * y + RN(-zero * y)) is within t * 1.5 * 2^-23 + ulp(t) +
    // 2^-24 * |zero * y| of RN(RN(x - zero) / s): 5 * 2^-20 + ... for t <= 16,
    // 2^-14 + ... for t <= 256.  The margin below is about 4x that.
    const float near_tie = 0.5f - ((BITS == 8 ? 0x1p-12f : 0x1p-16f) + 0x1p-22f * czmax);

    // codes, zero / scale of block g (whose rows are in t).  G = 32 (GT = 1):
    // the block's side area is kscale, kzero, vscale[4][32], vzero[4][32].
    // G > 32 (the split layout): it is vscale[NVG][32], vzero[NVG][32], and
    // the key zero / scale go to the key unit of the group (under the
    // segment policy: of the block), written by its first block only.
    constexpr bool SPLIT = GT > 1;
    constexpr int NVG = 4 / GT;                         // value groups per token
    constexpr int KUB = KSEG ? 1 : GT;                  // blocks per key unit
    auto store_block = [&](int64_t g) {
    uint8_t *blk = a.blocks + (stream * a.max_groups + g) * a.block_bytes;
    constexpr int cbytes = BITS * G * D / 8;
    _Float16 *side = (_Float16 *)(blk + 2 * cbytes);

    // zero / scale as fp16
    if (!IS_V) {
        // channels 8c..8c+7: lanes q = 0 store the scales, q = 1 the zeros
        // (0 and 0 for channels kept in fp16).
        if (q < 2) {
            float sk[8], zk[8];
#pragma unroll
            for (int k = 0; k < 8; k++) {
                const bool kept = OUT && ((omask >> k) & 1u);
                sk[k] = kept ? 0.0f : s[k];
                zk[k] = kept ? 0.0f : mn[k];
            }
            uint32_t w[4];
#pragma unroll
            for (int p = 0; p < 4; p++)
                w[p] = q == 0 ? pack_f16(sk[2 * p], sk[2 * p + 1]) : pack_f16(zk[2 * p], zk[2 * p + 1]);
            if constexpr (SPLIT) {
                if (g % KUB == 0) {
                    _Float16 *ku = (_Float16 *)(a.kside + (stream * a.max_kunits + g / KUB) * (4 * D));
                    *(uint4 *)(ku + q * D + 8 * c) = (uint4){w[0], w[1], w[2], w[3]};
                }
            } else {
                *(uint4 *)(side + q * D + 8 * c) = (uint4){w[0], w[1], w[2], w[3]};
            }
        }
        if constexpr (OUT) {
            // the block's outlier record: header (lane 0), each kept channel's
            // 32 fp16 values (the four lanes of its chunk, 8 rows each), zeros
            // in the unused slots (lanes 4o .. 4o + 3); no two stores overlap
            uint8_t *rec = a.outliers + (stream * a.max_groups + g) * kOutlierRecordBytes;
            if (l == 0)
                *(uint4 *)rec = (uint4){(uint32_t)och[0] | ((uint32_t)och[1] << 16),
                                        (uint32_t)och[2], 0u, 0u};
#pragma unroll
            for (int o = 0; o < kMaxKeyOutliers; o++) {
                if (o < a.n_out) {
                    if ((och[o] >> 3) == c) {
                        const int e = och[o] & 7;
                        _Float16 *dst = (_Float16 *)(rec + 16 + 64 * o);
#pragma unroll
                        for (int j = 0; j < 8; j++) {
                            // (a lane-dependent index into the 32-register tile
                            // would move it to scratch; into 8 copies it stays
                            // in registers)
                            float row[8];
#pragma unroll
                            for (int e2 = 0; e2 < 8; e2++) row[e2] = t.at(j, e2);
                            dst[tile_row<false>(j, q)] = (_Float16)row[e];
                        }
                    }
                } else if (l >= 4 * o && l < 4 * o + 4) {
                    *(uint4 *)(rec + 16 + 64 * o + 16 * (l - 4 * o)) = (uint4){0u, 0u, 0u, 0u};
                }
            }
            // the record's last 48 bytes (after the third slot) are zero too
            constexpr int kTail = 16 + 64 * kMaxKeyOutliers;
            if (l >= 12 && l < 12 + (kOutlierRecordBytes - kTail) / 16)
                *(uint4 *)(rec + kTail + 16 * (l - 12)) = (uint4){0u, 0u, 0u, 0u};
        }
    } else {
        // rows 4q..4q+3 (j < 4) and 16+4q.. (j >= 4) of value group c/4; the
        // four lanes of the quad store scale-low, scale-high, zero-low, zero-high.
        const int part = c & 3, jh = part & 1;
        float sv[8];
#pragma unroll
        for (int k = 0; k < 8; k++)     // rows past v_limit store scale 0 (their zero is +0)
            sv[k] = RING && g * G + tile_row<true>(k, q) >= a.v_limit ? 0.0f : s[k];
        // (selects on named values: an index into s[] / mn[] that depends on
        // the lane would move those arrays out of registers)
        const uint32_t s01 = pack_f16(sv[0], sv[1]), s23 = pack_f16(sv[2], sv[3]);
        const uint32_t s45 = pack_f16(sv[4], sv[5]), s67 = pack_f16(sv[6], sv[7]);
        const uint32_t z01 = pack_f16(mn[0], mn[1]), z23 = pack_f16(mn[2], mn[3]);
        const uint32_t z45 = pack_f16(mn[4], mn[5]), z67 = pack_f16(mn[6], mn[7]);
        const uint32_t w0 = part == 0 ? s01 : part == 1 ? s45 : part == 2 ? z01 : z45;
        const uint32_t w1 = part == 0 ? s23 : part == 1 ? s67 : part == 2 ? z23 : z67;
        if constexpr (SPLIT) {
            // slot gv of the value group of channels 32 (c / 4) ..: the quads
            // of one group hold the same pairs and store the same words
            *(uint2 *)(side + (part >> 1) * (NVG * G) + ((c >> 2) / GT) * G + 16 * jh + 4 * q) =
                (uint2){w0, w1};
        } else {
            *(uint2 *)(side + (2 + (part >> 1)) * D + (c >> 2) * G + 16 * jh + 4 * q) = (uint2){w0, w1};
        }
    }

    // Units u = 0..7 (key row j = u over channels kk; value channel e = u over
    // rows kk), parameters indexed by kk for keys and values alike.
    if constexpr (BITS == 8) {
        quantize_pack8<IS_V>(a, t, mn, s, y, cz, near_tie, fast_ok, blk, tr, OUT ? omask : 0u);
        return;
    }
    uint32_t unit[8];
#pragma unroll
    for (int u = 0; u < 8; u++) {
        float acc0 = 0.0f, acc1 = 0.0f, rmax = 0.0f;
#pragma unroll
        for (int kk = 0; kk < 8; kk++) {
            const float tq = IS_V ? t.fma(kk, u, y[kk], cz[kk]) : t.fma(u, kk, y[kk], cz[kk]);
            float cd = __builtin_rintf(tq);
            rmax = fmaxf(rmax, fabsf(tq - cd));
            if (OUT && !IS_V && ((omask >> kk) & 1u)) cd = 0.0f;    // kept in fp16
            if (kk < (BITS == 4 ? 2 : 1)) (kk ? acc1 : acc0) = cd;   // weight 1
            else if (BITS == 4 && (kk & 1)) acc1 = __builtin_fmaf(cd, unit_weight<BITS>(kk), acc1);
            else acc0 = __builtin_fmaf(cd, unit_weight<BITS>(kk), acc0);
        }
        if (!(rmax < near_tie) || !fast_ok) {
#pragma unroll
            for (int kk = 0; kk < 8; kk++) {
                const float x = IS_V ? t.at(kk, u) : t.at(u, kk);
                float cd = exact_code(x, mn[kk], s[kk], L);
                if (OUT && !IS_V && ((omask >> kk) & 1u)) cd = 0.0f;
                if (kk < (BITS == 4 ? 2 : 1)) (kk ? acc1 : acc0) = cd;
                else if (BITS == 4 && (kk & 1)) acc1 = __builtin_fmaf(cd, unit_weight<BITS>(kk), acc1);
                else acc0 = __builtin_fmaf(cd, unit_weight<BITS>(kk), acc0);
            }
        }
        unit[u] = BITS == 2 ? (uint32_t)acc0 : ((uint32_t)acc0 | ((uint32_t)acc1 << 16));
    }

    // Into packed order through LDS.  Target lane L keeps 4 (2-bit) or 8
    // (4-bit) dwords; the unit of its operand o sits in unit slot
    // 2*(o%4) + o/4 (16-bit slots at 2 bits, 32-bit slots at 4 bits).
    constexpr int DPL = 2 * BITS;
    if (!IS_V) {
        // key unit (row j = 4*jj + q, chunk c) -> lane (row%16) + 16*(c%4),
        // operand 4*(row/16) + c/4; rows j and j+4 share the target lane.
#pragma unroll
        for (int jj = 0; jj < 4; jj++) {
            const int L_ = 4 * jj + q + 16 * (c & 3);
            if (BITS == 2)
                tr[L_ * DPL + (c >> 2)] = unit[jj] | (unit[jj + 4] << 16);
            else
                *(uint2 *)&tr[L_ * DPL + 2 * (c >> 2)] = (uint2){unit[jj], unit[jj + 4]};
        }
    } else {
        // value unit (channel 8c + e over the lane's rows) -> lane
        // 8*(c%2) + e + 16q, operand c/2.
        const int o = c >> 1;
        const int slot = 2 * (o & 3) + (o >> 2);
#pragma unroll
        for (int e = 0; e < 8; e++) {
            const int L_ = 8 * (c & 1) + e + 16 * q;
            if (BITS == 2)
                ((uint16_t *)tr)[L_ * 2 * DPL + slot] = (uint16_t)unit[e];
            else
                tr[L_ * DPL + slot] = unit[e];
        }
    }
    __syncthreads();

    uint32_t outw[DPL];
    if (BITS == 2) {
        const uint4 d4 = *(const uint4 *)&tr[l * DPL];
        outw[0] = __builtin_amdgcn_perm(d4.y, d4.x, 0x05010400u);
        outw[1] = __builtin_amdgcn_perm(d4.w, d4.z, 0x05010400u);
        outw[2] = __builtin_amdgcn_perm(d4.y, d4.x, 0x07030602u);
        outw[3] = __builtin_amdgcn_perm(d4.w, d4.z, 0x07030602u);
    } else {
        const uint4 e0 = *(const uint4 *)&tr[l * DPL], e1 = *(const uint4 *)&tr[l * DPL + 4];
        const uint32_t ev[8] = {e0.x, e0.y, e0.z, e0.w, e1.x, e1.y, e1.z, e1.w};
#pragma unroll
        for (int o = 0; o < 8; o++) outw[o] = ev[2 * (o & 3) + (o >> 2)];
    }
    uint32_t *dst = (uint32_t *)(blk + (IS_V ? cbytes : 0));
#pragma unroll
    for (int w4 = 0; w4 < DPL / 4; w4++)
        *(uint4 *)&dst[w4 * 256 + 4 * l] =
            (uint4){outw[4 * w4], outw[4 * w4 + 1], outw[4 * w4 + 2], outw[4 * w4 + 3]};
    };

    if constexpr (IS_V || GT == 1 || KSEG) {
        store_block(g0);
    } else {
        store_block(g0 + GT - 1);
#pragma unroll 1
        for (int tt = GT - 2; tt >= 0; tt--) {
            load_tile<IS_V, RING>(a, stream, g0 + tt, t);
            __syncthreads();            // the previous block's LDS transpose is read
            store_block(g0 + tt);
        }
    }
}

// ===========================================================================
// Residual ring append: copy rows [tok_begin, tok_end) of the chunk into
// ring slot t % ring_cap.  16 bytes per thread.
// ===========================================================================
// The copy is split into 16-byte pieces of the flattened [streams][tokens]
// range of row pairs: a row pair (K and V) is 2 * D * esize / 16 pieces.
// The row's stream, token and slot are computed with 32-bit arithmetic where
// the range allows.  A ring append workgroup copies kRingThreads pieces, one
// per thread; the quantize launch that folds the copy in gives each of its
// copy workgroups the same kRingThreads pieces, kRingThreads / 64 per lane.
constexpr int kRingThreads = 256;

__device__ __forceinline__ void ring_copy_piece(const RingArgs &a, int64_t piece) {
    const int row_vec = D * a.esize / 16;                 // 16-byte pieces of one row
    const int per_row = 2 * row_vec;                      // K and V
    const int64_t ntok = a.tok_end - a.tok_begin;
    const int64_t rows = (int64_t)a.streams * ntok;
    const int64_t r = piece / per_row;
    if (r >= rows) return;
    const int e = (int)(piece % per_row);
    const int which = e >= row_vec;                       // 0: K, 1: V
    const int v = e - which * row_vec;
    int64_t stream, t;
    if (rows <= 0x7FFFFFFF) {
        const uint32_t r32 = (uint32_t)r, n32 = (uint32_t)ntok;
        stream = r32 / n32;
        t = a.tok_begin + (r32 - (uint32_t)stream * n32);
    } else {
        stream = r / ntok;
        t = a.tok_begin + (r - stream * ntok);
    }
    const uint32_t slot = a.ring_cap <= 0x7FFFFFFF && t <= 0xFFFFFFFFll
                              ? (uint32_t)t % (uint32_t)a.ring_cap
                              : (uint32_t)(t % a.ring_cap);
    const uint4 *src = (const uint4 *)((const uint8_t *)(which ? a.in_v : a.in_k) +
                                       (stream * a.n_new + (t - a.n_old)) * D * a.esize);
    uint4 *dst = (uint4 *)((uint8_t *)(which ? a.ring_v : a.ring_k) +
                           (stream * a.ring_cap + slot) * D * a.esize);
    dst[v] = src[v];
}

__global__ __launch_bounds__(kRingThreads) void ring_append_kernel(RingArgs a) {
    ring_copy_piece(a, (int64_t)blockIdx.x * kRingThreads + threadIdx.x);
}

// RING: the groups [group_begin, group_end) hold tokens appended earlier
// (read, at least in part, from the ring); otherwise every row comes from
// the new chunk.
// kinds = 3: per key group (GT blocks), task (1 + GT) i is the key group and
// the next GT tasks are the value blocks of the same tokens; kinds = 1 / 2:
// every task is a key group / a value block.
// Without RING, workgroups from a.quant_tasks on copy a.copy's ring rows.
// kinds = 4 (segment policy, KSEG): task 2i is the key block i with its
// segment's statistics, task 2i + 1 the value block i (groups of 32 * GT
// channels).
template <int BITS, typename T, bool RING, int GT, bool OUT, bool KSEG = false>
__global__ __launch_bounds__(64) void quantize_kernel(QuantizeArgs a) {
    __shared__ uint32_t tr[64 * 2 * BITS];
    const uint32_t task = blockIdx.x;
    if (task >= a.quant_tasks) {
        const int64_t first = (int64_t)(task - a.quant_tasks) * kRingThreads;
#pragma unroll
        for (int j = 0; j < kRingThreads / 64; j++)
            ring_copy_piece(a.copy, first + j * 64 + threadIdx.x);
        return;
    }
    const uint32_t nb = (uint32_t)(a.block_end - a.block_begin);
    int64_t stream, g;
    bool is_v;
    if (KSEG) {
        const uint32_t pair = task >> 1;
        stream = pair / nb;
        is_v = task & 1;
        g = a.block_begin + pair % nb;
    } else if (a.kinds == 3) {
        const uint32_t ngr = nb / GT, rest = task / (1 + GT), sub = task % (1 + GT);
        stream = rest / ngr;
        is_v = sub != 0;
        g = a.block_begin + (int64_t)(rest % ngr) * GT + (is_v ? sub - 1 : 0);
    } else if (a.kinds == 1) {
        const uint32_t ngr = nb / GT;
        stream = task / ngr;
        is_v = false;
        g = a.block_begin + (int64_t)(task % ngr) * GT;
    } else {
        stream = task / nb;
        is_v = true;
        g = a.block_begin + task % nb;
    }
    if (is_v) quantize_task<BITS, true, RING, T, GT, OUT>(a, stream, g, tr);
    else quantize_task<BITS, false, RING, T, GT, OUT, KSEG>(a, stream, g, tr);
}

// Segment policy: per-channel key minimum / maximum of the blocks [b0, b0 +
// seg_chunk_blocks) of one stream (one wavefront per (stream, chunk)), in
// float32 (exact for fp16 and fp32 inputs), to seg_partial.
template <typename T>
__global__ __launch_bounds__(64) void seg_stats_kernel(QuantizeArgs a) {
    const int64_t task = blockIdx.x;
    const int64_t stream = task / a.seg_chunks, ch = task % a.seg_chunks;
    const int64_t b0 = a.block_begin + ch * a.seg_chunk_blocks;
    const int64_t b1 = b0 + a.seg_chunk_blocks < a.block_end ? b0 + a.seg_chunk_blocks : a.block_end;
    const int l = threadIdx.x, q = l >> 4, c = l & 15;
    KPart<T> part;
    Tile<T> t;
#pragma unroll 1
    for (int64_t g = b0; g < b1; g++) {
        load_tile<false, true>(a, stream, g, t);
        kpart_add(t, part, g == b0);
    }
    float lo[8], hi[8];
    kpart_finish(part, lo, hi);
    float *dst = a.seg_partial + (stream * a.seg_chunks + ch) * 256 + 8 * c;
    if (q == 0) {
        *(float4 *)dst = (float4){lo[0], lo[1], lo[2], lo[3]};
        *(float4 *)(dst + 4) = (float4){lo[4], lo[5], lo[6], lo[7]};
    } else if (q == 1) {
        *(float4 *)(dst + 128) = (float4){hi[0], hi[1], hi[2], hi[3]};
        *(float4 *)(dst + 132) = (float4){hi[4], hi[5], hi[6], hi[7]};
    }
}

// The segment's statistics of one stream: minimum of the chunk minima and
// maximum of the chunk maxima (lane l: entries 4l .. 4l+3; minima for l < 32).
__global__ __launch_bounds__(64) void seg_reduce_kernel(QuantizeArgs a) {
    const int64_t stream = blockIdx.x;
    const int l = threadIdx.x;
    const bool is_max = l >= 32;
    const float *src = a.seg_partial + stream * a.seg_chunks * 256 + 4 * l;
    float4 acc = *(const float4 *)src;
    for (int ch = 1; ch < a.seg_chunks; ch++) {
        const float4 v = *(const float4 *)(src + ch * 256);
        if (is_max) {
            acc.x = fmax_(acc.x, v.x); acc.y = fmax_(acc.y, v.y);
            acc.z = fmax_(acc.z, v.z); acc.w = fmax_(acc.w, v.w);
        } else {
            acc.x = fmin_(acc.x, v.x); acc.y = fmin_(acc.y, v.y);
            acc.z = fmin_(acc.z, v.z); acc.w = fmin_(acc.w, v.w);
        }
    }
    *(float4 *)(a.seg_stats + stream * 256 + 4 * l) = acc;
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

// Reductions over the four 16-lane rows (lanes j, j+16, j+32, j+48).
__device__ __forceinline__ float xsum_rows(float v) {
    float a = v, b = v;
    swap_halves(a, b);
    float c = a + b, d = c;
    swap_rows(c, d);
    return c + d;
}
// NaN-propagating maximum (v_maximum3_f32): no operand quieting needed.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float xmax_rows(float v) {
    float a = v, b = v;
    swap_halves(a, b);
    float c = vmax(a, b), d = c;
    swap_rows(c, d);
    return vmax(c, d);
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
    } else if (BITS == 8) {
        // operand o = dwords 2o, 2o + 1; pair m in dword m / 2 at bits
        // 8 * (m % 2) and 16 + 8 * (m % 2)
#pragma unroll
        for (int m = 0; m < 4; m++) r[m] = ((m & 1) ? w[2 * o + (m >> 1)] >> 8 : w[2 * o + (m >> 1)]) & MASK;
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

__device__ __forceinline__ float load_q(const DecodeArgs &a, int64_t idx) {
    return a.q_is_f32 ? ((const float *)a.q)[idx] : (float)((const _Float16 *)a.q)[idx];
}

// q of query head hq as fp16 pairs in B-operand order: slice s, pair m ->
// channels 32s + 8*Gl + 2m, +1 (one 16-byte load per slice for fp16 q).
template <bool QF32>
__device__ __forceinline__ void load_q_operand(const void *qp, int64_t qrow, int Gl,
                                               h2 (&qB)[4][4]) {
    if constexpr (QF32) {
        const float *q = (const float *)qp + qrow + 8 * Gl;
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
        const _Float16 *q = (const _Float16 *)qp + qrow + 8 * Gl;
#pragma unroll
        for (int s = 0; s < 4; s++) split4(*(const uint4 *)(q + 32 * s), qB[s]);
    }
}

// Online softmax with a lazy maximum: a score may exceed the running maximum
// m_run by up to kSlack (log2 units) before the state is rescaled, so the
// cross-row reduction of the maximum and the rescale run only when some score
// passes m_thr = m_run + kSlack.  p is pre-divided by a further 2^kSlack,
// which keeps every fp16 p at or below 1.
constexpr int kSlack = 1;

template <int SB>
__device__ __forceinline__ constexpr int pair_shift(int m) {
    return kScaleLog2<SB>(m) + kSlack;
}

// ds_swizzle in bitmask mode (the LDS crossbar, no memory access): within
// each 32-lane half, lane i reads lane ((i & AND) | OR) ^ XOR.
template <int AND, int OR, int XOR>
__device__ __forceinline__ uint32_t swizzle(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, AND | (OR << 5) | (XOR << 10));
}
template <int XOR>
__device__ __forceinline__ float swizzle_xor(float v) {
    return __builtin_bit_cast(float, swizzle<31, 0, XOR>(__builtin_bit_cast(uint32_t, v)));
}

// One step over the 8 scores of a lane's column (two 16-token tiles): pair m
// holds tile m / 2, rows 2(m % 2), +1.  The 16 columns are GQ heads, each
// repeated 16 / GQ times, so the lanes h + GQ * m' (m' = 0..3) of a row hold
// the same scores: lane (j, row) computes p of pair own = (j / GQ) % 4 only,
// pre-divided by 2^pair_shift(own) (kScaleLog2<SB>(own) + kSlack), two
// exponentials instead of eight, and gathers the four pairs from those lanes.
// Returns p as fp16 pairs in value-operand order.  The unscaled sum of p runs
// on the matrix core: A holds the weights 2^pair_shift(m) in every row, so
// each row of Lsum carries the running sum of its column.  b0, b1: bits 0
// and 1 of own as masks of all ones or zeros; ps_own = pair_shift(own);
// nm_own caches -m_run - ps_own.
// (a & m) | (b & ~m): one v_bfi_b32, a lane-wise select by a mask of all ones
// or zeros that cannot become a branch.
__device__ __forceinline__ float bitsel(uint32_t m, float a, float b) {
    return __builtin_bit_cast(float, (__builtin_bit_cast(uint32_t, a) & m) |
                                         (__builtin_bit_cast(uint32_t, b) & ~m));
}

template <int SB, int GQ>
__device__ __forceinline__ void softmax_step(const f4 &S0, const f4 &S1, float cs, float kbl,
                                             uint32_t b0, uint32_t b1, float ps_own,
                                             float &m_run, float &m_thr, float &nm_own, f4 &Lsum,
                                             float (&vb)[4], f4 (&accV)[8], h2 (&P)[4]) {
    const float y = bitsel(b1, bitsel(b0, S1[2], S1[0]), bitsel(b0, S0[2], S0[0]));
    const float z = bitsel(b1, bitsel(b0, S1[3], S1[1]), bitsel(b0, S0[3], S0[1]));
    float mt = __builtin_fmaf(vmax(y, z), cs, kbl);   // this lane's maximum, log2 units
    if (__any(mt > m_thr)) {
        // the column's maximum: over the pair lanes of the row, then the rows
        mt = vmax(mt, swizzle_xor<GQ>(mt));
        mt = vmax(mt, swizzle_xor<2 * GQ>(mt));
        const float m_new = vmax(m_run, xmax_rows(mt));
        const float al = __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
        for (int o = 0; o < 8; o++) accV[o] *= al;
        Lsum *= al;
#pragma unroll
        for (int m = 0; m < 4; m++) vb[m] *= al;
        nm_own = -m_new - ps_own;
        m_run = m_new;
        m_thr = m_new + (float)kSlack;
    }
    const float nk = nm_own + kbl;
    const h2 d = {(_Float16)__builtin_amdgcn_exp2f(__builtin_fmaf(y, cs, nk)),
                  (_Float16)__builtin_amdgcn_exp2f(__builtin_fmaf(z, cs, nk))};
    const uint32_t du = __builtin_bit_cast(uint32_t, d);
    constexpr int AND = 16 | (GQ - 1);          // keep the head bits and the row parity
    P[0] = __builtin_bit_cast(h2, swizzle<AND, 0 * GQ, 0>(du));
    P[1] = __builtin_bit_cast(h2, swizzle<AND, 1 * GQ, 0>(du));
    P[2] = __builtin_bit_cast(h2, swizzle<AND, 2 * GQ, 0>(du));
    P[3] = __builtin_bit_cast(h2, swizzle<AND, 3 * GQ, 0>(du));
    h8 W;
#pragma unroll
    for (int m = 0; m < 4; m++) W[2 * m] = W[2 * m + 1] = (_Float16)(float)(1 << pair_shift<SB>(m));
    Lsum = __builtin_amdgcn_mfma_f32_16x16x32_f16(W, pack_h8(P), Lsum, 0, 0, 0);
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

// Order this wavefront's LDS accesses around a point (cross-lane exchange
// through LDS inside one wave; LDS executes a wave's operations in order).
__device__ __forceinline__ void lds_sync_wave() {
    asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
}

// 64 lanes x 16 bytes from global memory straight into LDS (one 1 KiB
// global_load_lds_dwordx4; LDS destination M0 + 16 * lane), and explicit waits
// on the vector-memory counter: the compiler's own wait insertion does not see
// these copies.  nt (wave-uniform) marks the lines non-temporal: data read
// once, which then does not displace what the caches hold (measured on a
// pure 400 MB read through this LDS ring: 5.97 -> 6.5 TB/s).
__device__ __forceinline__ void dma_1k(const uint8_t *src_lane, uint32_t lds_dst, bool nt = false) {
    // LDS destination: M0 + 16 * lane
    if (nt)
        asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off nt"
                     :
                     : "v"(src_lane), "s"(lds_dst)
                     : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                     :
                     : "v"(src_lane), "s"(lds_dst)
                     : "memory", "m0");
}

// Per-mille weight shift of decode splits between even and odd XCDs.
constexpr int64_t kXcdSkew = 20;

// Split items of the decode pass, in launch order: the grid's split items are
// cut into four quarters (quarter r holds (splits + 3 - r) / 4 splits of
// every stream, stream by stream, a stream's splits adjacent), so that each
// stream has splits in every quarter.  The quarters reach the compute units in
// turn, and a SIMD issues the wavefronts it received first ahead of the later
// ones: splits of earlier quarters get a larger share of their stream's
// groups (per mille of the average).
constexpr int64_t kQuarterWeight[4] = {1150, 1050, 950, 850};

__device__ __forceinline__ int64_t quarter_splits(int64_t splits, int r) {
    return (splits + 3 - r) / 4;
}

// Wavefront priority (s_setprio takes an immediate, 0..3).
__device__ __forceinline__ void set_prio(int p) {
    if (p >= 3) __builtin_amdgcn_s_setprio(3);
    else if (p == 2) __builtin_amdgcn_s_setprio(2);
    else if (p == 1) __builtin_amdgcn_s_setprio(1);
    else __builtin_amdgcn_s_setprio(0);
}

template <int N>
__device__ __forceinline__ void wait_vm() {
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// Residual items: tail_items per stream over the full-precision window
// [n_tail, n); item ti walks chunks [ti * step, (ti + 1) * step) of 32
// tokens, one at a time.  Each chunk's loads are issued
// together (one memory round trip per chunk), its softmax is local and is
// merged into the item's running state.

// p * v + acc with v one half of an fp16 pair, rounded once (v_fma_mix_f32).
// Written out so that the compiler keeps v packed instead of converting every
// pair to two fp32 registers up front.
__device__ __forceinline__ float fma_mix_lo(float p, h2 v, float acc) {
    float r;
    asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel_hi:[0,1,0]" : "=v"(r) : "v"(p), "v"(v), "v"(acc));
    return r;
}
__device__ __forceinline__ float fma_mix_hi(float p, h2 v, float acc) {
    float r;
    asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[0,1,0] op_sel_hi:[0,1,0]"
        : "=v"(r) : "v"(p), "v"(v), "v"(acc));
    return r;
}

__device__ __forceinline__ float readlane_f(float v, int lane) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// fp16 ring: scores on the matrix core (K rows and q are exact fp16).  The
// chunk's V rows are copied HBM -> LDS (8 KiB) alongside the K loads; p.V runs
// on the vector ALUs -- lane l owns channels 2l, 2l+1 and reads the chunk's p
// values (32 tokens x GQ heads) broadcast from LDS.
template <int GQ, bool QF32>
__device__ void decode_tail_f16(const DecodeArgs &a, int stream, int ti, uint8_t *lds) {
    const int l = threadIdx.x & 63;
    const int j = l & 15, Gl = l >> 4;
    const int h = j % GQ;
    const int b = stream / a.kv_heads, hk = stream % a.kv_heads;
    const int items = a.items;
    const int cap = (int)a.ring_cap;
    // uniform 64-bit bases + 32-bit per-lane byte offsets (one ring fits 4 GiB)
    const char *rkb = (const char *)a.ring_k + (int64_t)stream * a.ring_cap * D * 2;
    const char *rvb = (const char *)a.ring_v + (int64_t)stream * a.ring_cap * D * 2;
    const uint32_t vbase = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void *)lds;
    float *p_lds = (float *)(lds + G * D * 2);
    h2 qB[4][4];
    // (no wait here: the first chunk's loads overlap those of q, and the
    // compiler's wait before the first use of q also covers the copies)
    load_q_operand<QF32>(a.q, ((int64_t)b * a.q_heads + hk * GQ + h) * D, Gl, qB);
    // running state: per head (m, l) (wave-uniform) and the lane's two channels
    float Mr[GQ], Lr[GQ], O0[GQ], O1[GQ];
#pragma unroll
    for (int hh = 0; hh < GQ; hh++) { Mr[hh] = -INFINITY; Lr[hh] = 0.f; O0[hh] = O1[hh] = 0.f; }
    const int c_begin = ti * a.tail_chunk_step;
    const int c_end = c_begin + a.tail_chunk_step < a.tail_chunks ? c_begin + a.tail_chunk_step
                                                                   : a.tail_chunks;
    int slot0 = (int)((a.n_tail + (int64_t)G * c_begin) % a.ring_cap);
    for (int chunk = c_begin; chunk < c_end; chunk++) {
        const int64_t left = a.n_tokens - a.n_tail - (int64_t)G * chunk;
        const int cnt = left < G ? (int)left : G;        // >= 1
        // ring slot of chunk row r (rows past the end read the last valid
        // row; their scores are masked and their p is 0)
        auto slot = [&](int r) {
            const int s2 = slot0 + (r < cnt ? r : cnt - 1);
            return s2 >= cap ? s2 - cap : s2;
        };
        lds_sync_wave();   // the previous chunk's LDS reads are done
        const int cslot0 = slot0;
        // rows of tokens appended by this call come from the caller's buffer
        const int64_t tok0 = a.n_tail + (int64_t)G * chunk;
        const bool has_new = tok0 + cnt > a.in_from;                   // uniform
        auto new_row = [&](const void *base, int r) {
            const int rr = r < cnt ? r : cnt - 1;
            return (const char *)base + ((int64_t)stream * a.in_n + (tok0 + rr - a.in_from)) * D * 2;
        };
        // V rows -> LDS [32][D] fp16: copy i covers rows 4i .. 4i+3
#pragma unroll
        for (int i = 0; i < G / 4; i++) {
            const int r = 4 * i + Gl;
            const uint8_t *src = (const uint8_t *)rvb + (uint32_t)(slot(r) * D * 2 + 16 * j);
            if (has_new && tok0 + (r < cnt ? r : cnt - 1) >= a.in_from)
                src = (const uint8_t *)new_row(a.in_v, r) + 16 * j;
            dma_1k(src, __builtin_amdgcn_readfirstlane(vbase + 1024u * i));
        }
        uint4 kr[2][4];
#pragma unroll
        for (int t = 0; t < 2; t++) {
            const int r = 16 * t + j;
            const uint32_t off = (uint32_t)(slot(r) * D + 8 * Gl) * 2u;
            const char *kp = rkb + off;
            if (has_new && tok0 + (r < cnt ? r : cnt - 1) >= a.in_from)
                kp = new_row(a.in_k, r) + 16 * Gl;
#pragma unroll
            for (int s2 = 0; s2 < 4; s2++) kr[t][s2] = *(const uint4 *)(kp + 64u * s2);
        }
        if (has_new) {
            // the appended rows' keys into the ring (lanes of rows >= in_from)
            char *rkw = (char *)rkb;
#pragma unroll
            for (int t = 0; t < 2; t++) {
                const int r = 16 * t + j;
                if (r < cnt && tok0 + r >= a.in_from) {
                    char *dst = rkw + (uint32_t)(slot(r) * D + 8 * Gl) * 2u;
#pragma unroll
                    for (int s2 = 0; s2 < 4; s2++) *(uint4 *)(dst + 64u * s2) = kr[t][s2];
                }
            }
        }
        slot0 = slot0 + G >= cap ? slot0 + G - cap : slot0 + G;
        f4 S[2];
#pragma unroll
        for (int t = 0; t < 2; t++) {
            S[t] = (f4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s2 = 0; s2 < 4; s2++)
                S[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, kr[t][s2]),
                                                             pack_h8(qB[s2]), S[t], 0, 0, 0);
        }
        // lane (j, Gl) holds rows 16t + 4Gl + e of column j (query head j % GQ)
        float mt = -INFINITY;
#pragma unroll
        for (int t = 0; t < 2; t++)
#pragma unroll
            for (int e = 0; e < 4; e++) {
                if (16 * t + 4 * Gl + e >= cnt) S[t][e] = -INFINITY;
                mt = vmax(mt, S[t][e]);
            }
        const float m = xmax_rows(mt) * a.sm_log2;        // row 0 is always valid
        float ls = 0.f;
#pragma unroll
        for (int t = 0; t < 2; t++)
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(S[t][e], a.sm_log2, -m));
                ls += pv;
                if (j < GQ) p_lds[j * G + 16 * t + 4 * Gl + e] = pv;     // [head][token]
            }
        ls = xsum_rows(ls);
        wait_vm<0>();      // V copies landed
        lds_sync_wave();
        if (has_new) {
            // the appended rows' values into the ring, from LDS: 16 lanes per
            // row (slot0 already points at the next chunk: this chunk's slots
            // start at cslot0)
            const int r_first = a.in_from > tok0 ? (int)(a.in_from - tok0) : 0;
            char *rvw = (char *)rvb;
            for (int r = r_first + Gl; r < cnt; r += 4) {
                const int sr = cslot0 + r >= cap ? cslot0 + r - cap : cslot0 + r;
                *(uint4 *)(rvw + (uint32_t)(sr * D * 2 + 16 * j)) =
                    *(const uint4 *)(lds + r * D * 2 + 16 * j);
            }
        }
        // the lane's two channels of every row, then one accumulation chain per head
        const h2 *vl = (const h2 *)lds;
        h2 vr[G];
#pragma unroll
        for (int r = 0; r < G; r++) vr[r] = vl[r * (D / 2) + l];
#pragma unroll
        for (int hh = 0; hh < GQ; hh++) {
            float x0 = 0.f, x1 = 0.f;
#pragma unroll
            for (int r4 = 0; r4 < G / 4; r4++) {
                const float4 p4 = *(const float4 *)&p_lds[hh * G + 4 * r4];
                const float pq[4] = {p4.x, p4.y, p4.z, p4.w};
#pragma unroll
                for (int e = 0; e < 4; e++) {         // fp16 v enters the FMA directly
                    x0 = fma_mix_lo(pq[e], vr[4 * r4 + e], x0);
                    x1 = fma_mix_hi(pq[e], vr[4 * r4 + e], x1);
                }
            }
            // merge into the running state (head hh's (m, l) sit in lane hh)
            const float mc = readlane_f(m, hh), lc = readlane_f(ls, hh);
            const float mn = fmaxf(Mr[hh], mc);
            const float fo = __builtin_amdgcn_exp2f(Mr[hh] - mn);
            const float fc = __builtin_amdgcn_exp2f(mc - mn);
            O0[hh] = __builtin_fmaf(O0[hh], fo, x0 * fc);
            O1[hh] = __builtin_fmaf(O1[hh], fo, x1 * fc);
            Lr[hh] = __builtin_fmaf(Lr[hh], fo, lc * fc);
            Mr[hh] = mn;
        }
    }
#pragma unroll
    for (int hh = 0; hh < GQ; hh++) {
        const int64_t pi = ((int64_t)b * a.q_heads + hk * GQ + hh) * items + a.splits + ti;
        *(float2 *)&a.part_o[pi * D + 2 * l] = (float2){O0[hh], O1[hh]};
        if (l == 0) {
            a.part_ml[2 * pi] = Mr[hh];
            a.part_ml[2 * pi + 1] = Lr[hh];
        }
    }
}

// fp32 ring: one token per step on the vector ALUs (lane l owns channels 2l,
// 2l+1), online softmax in the log2 domain.
template <int GQ>
__device__ void decode_tail_f32(const DecodeArgs &a, int stream, int ti) {
    const int l = threadIdx.x & 63;
    const int b = stream / a.kv_heads, hk = stream % a.kv_heads;
    const int items = a.items;
    const int cap = (int)a.ring_cap;
    const int64_t t_begin = a.n_tail + (int64_t)G * ti * a.tail_chunk_step;
    const int64_t t_stop = t_begin + (int64_t)G * a.tail_chunk_step;
    const int64_t t_end = t_stop < a.n_tokens ? t_stop : a.n_tokens;
    int slot = (int)(t_begin % a.ring_cap);
    const float *rk = (const float *)a.ring_k + (int64_t)stream * a.ring_cap * D;
    const float *rv = (const float *)a.ring_v + (int64_t)stream * a.ring_cap * D;
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
    for (int64_t t = t_begin; t < t_end; t++) {
        const int64_t row = (int64_t)slot * D + 2 * l;
        slot = slot + 1 == cap ? 0 : slot + 1;
        float k0, k1, v0, v1;
        if (t >= a.in_from) {
            // a row appended by this call: from the caller's buffer, and into the ring
            const int64_t src = ((int64_t)stream * a.in_n + (t - a.in_from)) * D + 2 * l;
            const float2 kk = *(const float2 *)((const float *)a.in_k + src);
            const float2 vv = *(const float2 *)((const float *)a.in_v + src);
            *(float2 *)((float *)rk + row) = kk;
            *(float2 *)((float *)rv + row) = vv;
            k0 = kk.x; k1 = kk.y; v0 = vv.x; v1 = vv.y;
        } else {
            k0 = rk[row]; k1 = rk[row + 1]; v0 = rv[row]; v1 = rv[row + 1];
        }
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
        const int64_t pi = ((int64_t)b * a.q_heads + hk * GQ + h) * items + a.splits + ti;
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
    static constexpr int NST = BITS == 2 ? 3 : 2;       // stages (8 bits: 9 KiB groups)
};

// LDS bytes of one pipeline stage: the block, and with outlier-aware keys
// (OUT) the block's 256-byte outlier record after it.
template <int BITS, bool OUT>
__device__ __forceinline__ constexpr int stage_bytes() {
    return Pipe<BITS>::BB + (OUT ? kOutlierRecordBytes : 0);
}
// Stages of the decode pipeline: with records, two at 2 bits as well, so
// that a wavefront's LDS stays within 10 KiB (16 per compute unit).  DEEP
// (4 bits, long passes): three, 15 KiB, 10 wavefronts per compute unit.
template <int BITS, bool OUT, bool DEEP = false>
__device__ __forceinline__ constexpr int decode_stages() {
    return OUT ? 2 : DEEP ? 3 : Pipe<BITS>::NST;
}
// LDS of a decode wavefront besides q: the stages, and at least what a
// residual item uses (32 fp16 value rows, then p of 4 heads x 32 tokens).
template <int BITS, bool OUT, bool DEEP = false>
__device__ __forceinline__ constexpr int decode_lds_bytes() {
    constexpr int st = decode_stages<BITS, OUT, DEEP>() * stage_bytes<BITS, OUT>();
    constexpr int tail = G * D * 2 + 4 * G * 4;
    return st > tail ? st : tail;
}

// 64 lanes x 4 bytes from global memory straight into LDS (M0 + 4 * lane).
__device__ __forceinline__ void dma_256(const uint8_t *src_lane, uint32_t lds_dst, bool nt = false) {
    if (nt)
        asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off nt"
                     :
                     : "v"(src_lane), "s"(lds_dst)
                     : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off"
                     :
                     : "v"(src_lane), "s"(lds_dst)
                     : "memory", "m0");
}

// One group into an LDS stage.  G = 32: the whole block (and with OUT its
// outlier record after it).  Split layout (SPLIT): the block's codes, then
// its key unit ku (512 bytes) at the offset where a G = 32 block has its key
// scale and zero, then its value pairs (vbytes = 128 * value slots per
// token: lanes past them copy the first ones again, into LDS the stage does
// not use), so that the stage reads the same way in both layouts.
template <int BITS, bool OUT = false, bool SPLIT = false>
__device__ __forceinline__ void issue_group(const uint8_t *blk, const uint8_t *rec, uint32_t stage,
                                            int l, bool nt = false, const uint8_t *ku = nullptr,
                                            int vlanes = 64) {
    asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");   // prior reads of the stage done
    if constexpr (SPLIT) {
        constexpr int CB2 = 2 * Pipe<BITS>::CB;
#pragma unroll
        for (int c = 0; c < CB2 / 1024; c++)
            dma_1k(blk + c * 1024 + 16 * l, __builtin_amdgcn_readfirstlane(stage + c * 1024), nt);
        dma_256(ku + 4 * l, __builtin_amdgcn_readfirstlane(stage + CB2), nt);
        dma_256(ku + 256 + 4 * l, __builtin_amdgcn_readfirstlane(stage + CB2 + 256), nt);
        dma_256(blk + CB2 + 4 * (l & (vlanes - 1)), __builtin_amdgcn_readfirstlane(stage + CB2 + 512),
                nt);
    } else {
#pragma unroll
        for (int c = 0; c < Pipe<BITS>::DPG; c++)
            dma_1k(blk + c * 1024 + 16 * l, __builtin_amdgcn_readfirstlane(stage + c * 1024), nt);
        if constexpr (OUT)
            dma_256(rec + 4 * l, __builtin_amdgcn_readfirstlane(stage + Pipe<BITS>::BB), nt);
    }
}

// Wait until at most `r` groups (issued after the one needed) are in flight.
template <int BITS, bool OUT = false, bool SPLIT = false>
__device__ __forceinline__ void wait_groups_after(int r) {
    constexpr int P = SPLIT ? 2 * Pipe<BITS>::CB / 1024 + 3 : Pipe<BITS>::DPG + (OUT ? 1 : 0);
    if (r >= 3) wait_vm<3 * P>();
    else if (r == 2) wait_vm<2 * P>();
    else if (r == 1) wait_vm<P>();
    else wait_vm<0>();
}

template <int BITS, int GQ, bool QF32, bool OUT = false, bool DEEP = false, bool SPLIT = false>
__device__ void decode_split(const DecodeArgs &a, int stream, int sp, uint8_t *pipe,
                             uint4 *q_lds) {
    using PP = Pipe<BITS>;
    constexpr int SB = stage_bytes<BITS, OUT>();
    constexpr int NST = decode_stages<BITS, OUT, DEEP>();
    constexpr int DPL = 2 * BITS;              // code dwords per lane
    const int l = threadIdx.x & 63;
    const int j = l & 15, Gl = l >> 4;
    const int h = j % GQ;
    const int cg = (j / GQ) & 3;
    const int b = stream / a.kv_heads, hk = stream % a.kv_heads;
    const int hq = hk * GQ + h;
    const int items = a.items;
    const int64_t ng = a.n_quant / G;
    // The stream's ng groups are shared among its splits in proportion to a
    // weight per split: the weight of the split's quarter of the grid
    // (kQuarterWeight) times an XCD factor.  Workgroups go to the eight XCDs
    // in turn (block b to XCD b mod 8), and on MI355X the odd-numbered XCDs
    // stream slower than the even ones (4-10 % with cached copies, about half
    // that with the non-temporal ones), so splits whose block is odd get
    // kXcdSkew per mille less than the average and even ones that much more.
    // Any weights give the same groups overall, so results do not depend on
    // them.  Split k of quarter r is block tail + streams * (splits before
    // quarter r) + stream * (quarter's splits) + (k - splits before r).
    // (Block numbers stay below 2^31, the launch checks it, so the parities
    // are taken in 32 bits; a split's share and the weights in 64.  The
    // shares' quotients are IEEE double divisions of integers below 2^53,
    // which truncate to the integer quotient: the rounding error, at most
    // quotient * 2^-53, is smaller than 1 / wsum, the least distance of a
    // fraction with that denominator from an integer.  A scalar 64-bit
    // division costs over a hundred instructions, and a compute unit's
    // scalar unit serves its 16 wavefronts' prologues in turn.)
    constexpr int WE = 1000 + (int)kXcdSkew, WO = 1000 - (int)kXcdSkew;
    const int streams32 = a.batch * a.kv_heads;
    const int tail_blocks = streams32 * (a.tail_items + a.mixed_items);
    auto cum = [&](int k) {                             // weight of splits [0, k)
        int64_t c = 0;
        int k0 = 0;
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const int u = (a.splits + 3 - r) >> 2;      // quarter_splits
            const int m = k - k0 < 0 ? 0 : k - k0 > u ? u : k - k0;
            const int base = tail_blocks + streams32 * k0 + stream * u;
            const int odd = ((base + m) >> 1) - (base >> 1);
            c += kQuarterWeight[r] * (int64_t)((m - odd) * WE + odd * WO);
            k0 += u;
        }
        return c;
    };
    const double wsum = (double)cum(a.splits);
    const int64_t g0 = (int64_t)((double)(ng * cum(sp)) / wsum);
    const int64_t g1 = (int64_t)((double)(ng * cum(sp + 1)) / wsum);
    const int n_g = (int)(g1 - g0);             // groups of this split

    const uint8_t *sblk = a.blocks + ((int64_t)stream * a.max_groups + g0) * a.block_bytes;
    const uint8_t *srec = OUT ? a.outliers + ((int64_t)stream * a.max_groups + g0) * kOutlierRecordBytes
                              : nullptr;
    const int64_t bstride = SPLIT ? a.block_bytes : PP::BB;
    // split layout: the key unit of group g0 + i, and the value-pair lanes
    const uint8_t *skside = a.side.kside + (int64_t)stream * a.side.max_kunits * (4 * D);
    auto kunit = [&](int i) { return skside + ((g0 + i) >> a.side.kunit_shift) * (4 * D); };
    const int vlanes = 32 * a.side.nvs;
    const uint32_t pbase = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void *)pipe;
    const bool nt = a.nt != 0;                  // the pass streams more than the caches keep
    // q of the lane's head in B-operand order, and the unscaled fp16 q of the
    // GQ heads for LDS (16 bytes per lane, head (l/16) % GQ, channels
    // 8*(l%16)..+7: B operand of the key-zero product).  The first copies go
    // out before either is used, so the prologue costs one memory round trip.
    // (The compiler's own wait before the first use of q also covers the
    // copies, which it does not see: loads complete in order.)
    h2 qB[4][4];
    load_q_operand<QF32>(a.q, ((int64_t)b * a.q_heads + hq) * D, Gl, qB);
    uint4 uq;
    {
        const int64_t qoff = ((int64_t)b * a.q_heads + hk * GQ + (l >> 4) % GQ) * D + 8 * (l & 15);
        if constexpr (QF32) {
            const float *qf = (const float *)a.q + qoff;
            const float4 x0 = *(const float4 *)qf, x1 = *(const float4 *)(qf + 4);
            h2 t0 = {(_Float16)x0.x, (_Float16)x0.y}, t1 = {(_Float16)x0.z, (_Float16)x0.w};
            h2 t2 = {(_Float16)x1.x, (_Float16)x1.y}, t3 = {(_Float16)x1.z, (_Float16)x1.w};
            uq.x = __builtin_bit_cast(uint32_t, t0); uq.y = __builtin_bit_cast(uint32_t, t1);
            uq.z = __builtin_bit_cast(uint32_t, t2); uq.w = __builtin_bit_cast(uint32_t, t3);
        } else {
            uq = *(const uint4 *)((const _Float16 *)a.q + qoff);
        }
    }
    // stage ring: `is` is the stage the next copy goes to, `rs` the stage read
    int issued = 0, is = 0, rs = 0;
    for (; issued < NST - 1 && issued < n_g; issued++) {
        issue_group<BITS, OUT, SPLIT>(sblk + (int64_t)issued * bstride,
                                      OUT ? srec + (int64_t)issued * kOutlierRecordBytes : nullptr,
                                      pbase + (uint32_t)is * SB, l, nt,
                                      SPLIT ? kunit(issued) : nullptr, vlanes);
        is = is + 1 == NST ? 0 : is + 1;
    }
    // first uses of q: after the copies above (volatile asm keeps the order)
#pragma unroll
    for (int s = 0; s < 4; s++)
#pragma unroll
        for (int m = 0; m < 4; m++) asm volatile("" : "+v"(qB[s][m]));
    asm volatile("" : "+v"(uq.x), "+v"(uq.y), "+v"(uq.z), "+v"(uq.w));
    q_lds[l] = uq;
#pragma unroll
    for (int m = 0; m < 4; m++) {
        const _Float16 dn = (_Float16)(1.0f / (float)(1 << kScaleLog2<BITS>(m)));
        const h2 d2 = {dn, dn};
#pragma unroll
        for (int s = 0; s < 4; s++) qB[s][m] = qB[s][m] * d2;
    }
    const float cs = a.sm_log2 * kTwo24;        // score units -> log2 units

    float m_run = -INFINITY, m_thr = -INFINITY;
    f4 Lsum = (f4){0.f, 0.f, 0.f, 0.f};
    float nm_own = INFINITY, vb[4] = {0.f, 0.f, 0.f, 0.f};
    const int own = (j / GQ) & 3;               // the pair of p this lane computes
    const uint32_t ob0 = (own & 1) ? ~0u : 0u, ob1 = (own & 2) ? ~0u : 0u;
    const float ps_own = (float)(kScaleLog2<BITS>(own) + kSlack);
    // value pairs of the lane's channel group cg, in 8-byte units from the
    // side area: slot cg >> vsh of nvs (tokens 4 Gl .., +4 for 16 + 4 Gl ..)
    const int vsi = 64 + 8 * (cg >> (SPLIT ? a.side.vsh : 0)) + Gl;
    const int vzi = vsi + 8 * (SPLIT ? a.side.nvs : 4);
    f4 accV[8];
#pragma unroll
    for (int o = 0; o < 8; o++) accV[o] = (f4){0.f, 0.f, 0.f, 0.f};

    // The SIMD issues the oldest of its wavefronts first, so with equal
    // shares the first-dispatched splits finish long before the last ones and
    // the end of the pass runs with few copies in flight.  Each split lowers
    // its priority as it advances (3 over its first quarter, down to 0 over
    // its last): lagging wavefronts are issued first and the splits finish
    // closer together.  (Results do not depend on it.)
    int prio = 3, next_at = (n_g + 3) / 4;     // priority 3 - floor(4 g / n_g)
    set_prio(prio);
    for (int g = 0; g < n_g; g++) {
        if (g == next_at) {
            while (prio > 0 && g == next_at) {
                prio--;
                next_at = (n_g * (4 - prio) + 3) / 4;
            }
            set_prio(prio);
        }
        if (issued < n_g) {
            issue_group<BITS, OUT, SPLIT>(sblk + (int64_t)issued * bstride,
                                          OUT ? srec + (int64_t)issued * kOutlierRecordBytes : nullptr,
                                          pbase + (uint32_t)is * SB, l, nt,
                                          SPLIT ? kunit(issued) : nullptr, vlanes);
            is = is + 1 == NST ? 0 : is + 1;
            issued++;
        }
        wait_groups_after<BITS, OUT, SPLIT>(issued - 1 - g);
        const uint8_t *stg = pipe + rs * SB;
        rs = rs + 1 == NST ? 0 : rs + 1;
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
        if constexpr (OUT) {
            // key channels kept in fp16: their codes, scale and zero are 0, so
            // add q . K over them from the record (exact fp16 products; the
            // scores here are in units of 2^24)
            const uint2 idx = *(const uint2 *)(stg + PP::BB);    // channel[0..2]
            const int ch[kMaxKeyOutliers] = {(int)(idx.x & 0xFFFFu), (int)(idx.x >> 16),
                                             (int)(idx.y & 0xFFFFu)};
            const _Float16 *rval = (const _Float16 *)(stg + PP::BB + 16);
            const _Float16 *q16 = (const _Float16 *)q_lds;      // [head][channel]
#pragma unroll
            for (int o = 0; o < kMaxKeyOutliers; o++) {
                if (o < a.n_out) {
                    const float qo = (float)q16[h * D + ch[o]] * kTwoM24;
                    const h2 *v0 = (const h2 *)(rval + G * o + 4 * Gl);        // tokens 4Gl + e
                    const h2 *v1 = (const h2 *)(rval + G * o + 16 + 4 * Gl);   // 16 + 4Gl + e
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        S0[e] = __builtin_fmaf(qo, (float)v0[e >> 1][e & 1], S0[e]);
                        S1[e] = __builtin_fmaf(qo, (float)v1[e >> 1][e & 1], S1[e]);
                    }
                }
            }
        }
        h2 P[4];
        softmax_step<BITS, GQ>(S0, S1, cs, Sk[0] * a.sm_log2, ob0, ob1, ps_own, m_run, m_thr,
                               nm_own, Lsum, vb, accV, P);
        h2 vs[4], vz[4], ps[4];
        {
            const uint2 *s2 = (const uint2 *)side;
            const uint2 a0 = s2[vsi], a1 = s2[vsi + 4];
            const uint2 z0 = s2[vzi], z1 = s2[vzi + 4];
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
    vbt *= (float)(1 << kSlack);
    const int64_t pi = ((int64_t)b * a.q_heads + hq) * items + sp;
    store_partial<GQ>(a, pi, l, accV, kTwo24 * (float)(1 << kSlack), xsum_rows(vbt), m_run,
                      Lsum[0]);
}

// Position of the code of (token t, channel c) of a group in its code area:
// dword index and bit, following the operand layout the quantizer writes
// (keys: lane (t % 16) + 16 ((c % 32) / 8), operand 4 (t / 16) + c / 32,
// kk = c % 8; values: lane (c % 16) + 16 ((t % 16) / 4), operand c / 16,
// kk = t % 4 + 4 (t / 16)).
template <int BITS>
__device__ __forceinline__ void code_pos(bool is_v, int t, int c, int &dw, int &bit) {
    const int lane = is_v ? (c & 15) + 16 * ((t & 15) >> 2) : (t & 15) + 16 * ((c >> 3) & 3);
    const int o = is_v ? c >> 4 : 4 * (t >> 4) + (c >> 5);
    const int kk = is_v ? (t & 3) + 4 * (t >> 4) : c & 7;
    const int h = kk & 1;
    int w, i;
    if (BITS == 2) { w = o >> 1; i = 4 * (o & 1) + (kk >> 1); }
    else if (BITS == 4) { w = o; i = kk >> 1; }
    else { w = 2 * o + (kk >> 2); i = (kk >> 1) & 1; }
    dw = (w >> 2) * 256 + 4 * lane + (w & 3);
    bit = 16 * h + BITS * i;
}

// Paper policy ([RV] 3.2.2-3.2.3, Algorithm 1): keys are quantized R tokens
// at a time and values one token at a time, so the groups [n_quant / G,
// n_tail / G) have key codes while their value codes stop at n_vquant (at
// most R / G + 1 groups per stream).  Item mi of a stream takes mixed_step of
// them.  Per group: the block is copied into LDS and the scores come from the
// matrix core exactly as in decode_split (codes, q * kscale as hi + lo, the
// key-zero bias); the softmax is local to the group and merged into the
// item's running state like a residual chunk; p.V runs on the vector ALUs,
// lane l owning channels 2l, 2l+1, with V-hat = code * scale, then + zero,
// in float32 for tokens below n_vquant and the ring's rows for the others.
// The items are blocks of decode_kernel's launch (after the residual items,
// before the splits) and use its LDS: the block, p, and kMixedRowBytes of
// ring rows, so that the item holds no more registers than a split item.
constexpr int kMixedRowBytes = 4096;

template <int BITS, int GQ, bool RF32, bool QF32, bool OUT, bool SPLIT = false>
__device__ void decode_mixed_t(const DecodeArgs &a, int stream, int mi, uint8_t *lds,
                               uint4 *q_lds) {
    using PP = Pipe<BITS>;
    constexpr int SB = stage_bytes<BITS, OUT>();
    constexpr uint32_t M1 = (1u << BITS) - 1u;
    const int l = threadIdx.x & 63;
    const int j = l & 15, Gl = l >> 4;
    const int h = j % GQ;
    const int b = stream / a.kv_heads, hk = stream % a.kv_heads;
    const char *rvb = (const char *)a.ring_v + (int64_t)stream * a.ring_cap * D * (RF32 ? 4 : 2);
    const uint32_t lbase = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void *)lds;
    float *p_lds = (float *)(lds + SB);               // [G][GQ]
    // q of the lane's head is loaded here, the unscaled q for LDS after the
    // first group's copies and value-row loads; both are first used after
    // those, so the item waits one memory round trip for all of them (loads
    // complete in order)
    h2 qB[4][4];
    load_q_operand<QF32>(a.q, ((int64_t)b * a.q_heads + hk * GQ + h) * D, Gl, qB);
    const int64_t qoff = ((int64_t)b * a.q_heads + hk * GQ + (l >> 4) % GQ) * D + 8 * (l & 15);
    const float cs = a.sm_log2 * kTwo24;
    float Mr[GQ], Lr[GQ], O0[GQ], O1[GQ];
#pragma unroll
    for (int hh = 0; hh < GQ; hh++) { Mr[hh] = -INFINITY; Lr[hh] = 0.f; O0[hh] = O1[hh] = 0.f; }
    const int c0 = 2 * l, cgv = c0 / G;
    // value pairs of channel group cgv (fp16 index from the side area)
    const int vsf = 2 * D + G * (cgv >> a.side.vsh), vzf = vsf + G * a.side.nvs;
    const int g_begin = mi * a.mixed_step;
    const int g_end = g_begin + a.mixed_step < a.mixed_groups ? g_begin + a.mixed_step
                                                               : a.mixed_groups;
    for (int gi = g_begin; gi < g_end; gi++) {
        const int64_t g = a.n_quant / G + gi;
        const uint8_t *blk = a.blocks + ((int64_t)stream * a.max_groups + g) * a.block_bytes;
        lds_sync_wave();            // the previous group's LDS reads are done
        issue_group<BITS, OUT, SPLIT>(
            blk, OUT ? a.outliers + ((int64_t)stream * a.max_groups + g) * kOutlierRecordBytes : nullptr,
            lbase, l, false,
            a.side.kside + ((int64_t)stream * a.side.max_kunits + (g >> a.side.kunit_shift)) * (4 * D),
            32 * a.side.nvs);
        if (gi == g_begin) {
            uint4 uq;
            if constexpr (QF32) {
                const float *qf = (const float *)a.q + qoff;
                const float4 x0 = *(const float4 *)qf, x1 = *(const float4 *)(qf + 4);
                h2 t0 = {(_Float16)x0.x, (_Float16)x0.y}, t1 = {(_Float16)x0.z, (_Float16)x0.w};
                h2 t2 = {(_Float16)x1.x, (_Float16)x1.y}, t3 = {(_Float16)x1.z, (_Float16)x1.w};
                uq.x = __builtin_bit_cast(uint32_t, t0); uq.y = __builtin_bit_cast(uint32_t, t1);
                uq.z = __builtin_bit_cast(uint32_t, t2); uq.w = __builtin_bit_cast(uint32_t, t3);
            } else {
                uq = *(const uint4 *)((const _Float16 *)a.q + qoff);
            }
            // first uses of q: after the copies and loads above (volatile asm
            // keeps the order; q is not touched before this point)
#pragma unroll
            for (int s2 = 0; s2 < 4; s2++)
#pragma unroll
                for (int m = 0; m < 4; m++) asm volatile("" : "+v"(qB[s2][m]));
            q_lds[l] = uq;
#pragma unroll
            for (int m = 0; m < 4; m++) {
                const _Float16 dn = (_Float16)(1.0f / (float)(1 << kScaleLog2<BITS>(m)));
                const h2 d2 = {dn, dn};
#pragma unroll
                for (int s2 = 0; s2 < 4; s2++) qB[s2][m] = qB[s2][m] * d2;
            }
        }
        wait_vm<0>();
        lds_sync_wave();
        const uint8_t *stg = lds;
        const uint4 *side = (const uint4 *)(stg + 2 * PP::CB);
        uint32_t kc[2 * BITS];
#pragma unroll
        for (int w4 = 0; w4 < BITS / 2; w4++) {
            const uint4 u = *(const uint4 *)(stg + w4 * 1024 + 16 * l);
            kc[4 * w4] = u.x; kc[4 * w4 + 1] = u.y; kc[4 * w4 + 2] = u.z; kc[4 * w4 + 3] = u.w;
        }
        f4 Sk = (f4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s2 = 0; s2 < 4; s2++)
            Sk = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                __builtin_bit_cast(h8, side[16 + 4 * s2 + Gl]),
                __builtin_bit_cast(h8, q_lds[16 * (j % GQ) + 4 * s2 + Gl]), Sk, 0, 0, 0);
        f4 S[2] = {(f4){0.f, 0.f, 0.f, 0.f}, (f4){0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int s2 = 0; s2 < 4; s2++) {
            h2 ks[4], qh[4], ql[4];
            split4(side[4 * s2 + Gl], ks);
#pragma unroll
            for (int m = 0; m < 4; m++) {
                qh[m] = qB[s2][m] * ks[m];
                ql[m] = __builtin_elementwise_fma(qB[s2][m], ks[m], -qh[m]);
            }
            const h8 A0 = unpack_operand<BITS>(kc, s2), A1 = unpack_operand<BITS>(kc, 4 + s2);
            const h8 Bh = pack_h8(qh), Bl = pack_h8(ql);
            S[0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A0, Bh, S[0], 0, 0, 0);
            S[1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A1, Bh, S[1], 0, 0, 0);
            S[0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A0, Bl, S[0], 0, 0, 0);
            S[1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A1, Bl, S[1], 0, 0, 0);
        }
        if constexpr (OUT) {
            // key channels kept in fp16: q . K over them from the record, in
            // the scores' units of 2^24 (as in decode_split)
            const uint2 idx = *(const uint2 *)(stg + PP::BB);
            const int ch[kMaxKeyOutliers] = {(int)(idx.x & 0xFFFFu), (int)(idx.x >> 16),
                                             (int)(idx.y & 0xFFFFu)};
            const _Float16 *rval = (const _Float16 *)(stg + PP::BB + 16);
            const _Float16 *q16 = (const _Float16 *)q_lds;      // [head][channel]
#pragma unroll
            for (int o = 0; o < kMaxKeyOutliers; o++) {
                if (o < a.n_out) {
                    const float qo = (float)q16[h * D + ch[o]] * kTwoM24;
                    const h2 *v0 = (const h2 *)(rval + G * o + 4 * Gl);
                    const h2 *v1 = (const h2 *)(rval + G * o + 16 + 4 * Gl);
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        S[0][e] = __builtin_fmaf(qo, (float)v0[e >> 1][e & 1], S[0][e]);
                        S[1][e] = __builtin_fmaf(qo, (float)v1[e >> 1][e & 1], S[1][e]);
                    }
                }
            }
        }
        // lane (j, Gl) holds tokens 16t + 4Gl + e of column j (head j % GQ),
        // in log2 units after the scale and the key-zero bias
        const float kbl = Sk[0] * a.sm_log2;
        float mt = -INFINITY;
#pragma unroll
        for (int t = 0; t < 2; t++)
#pragma unroll
            for (int e = 0; e < 4; e++) {
                S[t][e] = __builtin_fmaf(S[t][e], cs, kbl);
                mt = vmax(mt, S[t][e]);
            }
        const float m = xmax_rows(mt);
        float ls = 0.f;
#pragma unroll
        for (int t = 0; t < 2; t++)
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const float pv = __builtin_amdgcn_exp2f(S[t][e] - m);
                ls += pv;
                if (j < GQ) p_lds[(16 * t + 4 * Gl + e) * GQ + j] = pv;  // [token][head]
            }
        ls = xsum_rows(ls);
        lds_sync_wave();
        // p . V, lane l owning channels c0, c0 + 1: rows below n_vquant from
        // their codes (V-hat = code * scale, then + zero, in float32), the
        // others from the ring.  Those are copied into LDS 4 KiB at a time
        // (16 fp16 or 8 fp32 rows; a group's rows are contiguous in the ring,
        // whose size and the group's first slot are multiples of G) and read
        // a row at a time, so that they hold no registers; each head sums its
        // rows in order.
        constexpr int RB = RF32 ? 4 : 2;
        constexpr int CR = kMixedRowBytes / (D * RB);       // rows per copy
        const uint32_t rows_lds = lbase + (uint32_t)(SB + GQ * G * 4);
        const uint8_t *rows = lds + SB + GQ * G * 4;
        const uint8_t *rsrc = (const uint8_t *)rvb + (g * G) % a.ring_cap * D * RB;
        const int64_t ncv = a.n_vquant - g * G;
        const int nc = ncv < 0 ? 0 : ncv > G ? G : (int)ncv;  // rows with codes
        const uint32_t *vcode = (const uint32_t *)(stg + PP::CB);
        const _Float16 *sd = (const _Float16 *)(stg + 2 * PP::CB);
        float x0[GQ], x1[GQ];
#pragma unroll
        for (int hh = 0; hh < GQ; hh++) x0[hh] = x1[hh] = 0.f;
        for (int r0 = 0; r0 < G; r0 += CR) {
            if (r0 + CR > nc) {
                lds_sync_wave();            // the previous rows' LDS reads are done
#pragma unroll
                for (int c = 0; c < kMixedRowBytes / 1024; c++)
                    dma_1k(rsrc + r0 * D * RB + c * 1024 + 16 * l,
                           __builtin_amdgcn_readfirstlane(rows_lds + c * 1024));
                wait_vm<0>();
            }
#pragma unroll 2
            for (int i = 0; i < CR; i++) {
                const int r = r0 + i;
                float vx, vy;
                if (r < nc) {
#pragma clang fp contract(off)
                    int dv0, bv0, dv1, bv1;
                    code_pos<BITS>(true, r, c0, dv0, bv0);
                    code_pos<BITS>(true, r, c0 + 1, dv1, bv1);
                    const float vs = (float)sd[vsf + r];
                    const float vz = (float)sd[vzf + r];
                    vx = (float)((vcode[dv0] >> bv0) & M1) * vs + vz;
                    vy = (float)((vcode[dv1] >> bv1) & M1) * vs + vz;
                } else if constexpr (RF32) {
                    const float2 f = *(const float2 *)(rows + (i * D + c0) * 4);
                    vx = f.x;
                    vy = f.y;
                } else {
                    const h2 hv = *(const h2 *)(rows + (i * D + c0) * 2);
                    vx = (float)hv[0];
                    vy = (float)hv[1];
                }
                float pr[GQ];
                if constexpr (GQ == 4) {
                    const float4 p4 = *(const float4 *)&p_lds[4 * r];
                    pr[0] = p4.x; pr[1] = p4.y; pr[2] = p4.z; pr[3] = p4.w;
                } else if constexpr (GQ == 2) {
                    const float2 p2 = *(const float2 *)&p_lds[2 * r];
                    pr[0] = p2.x; pr[1] = p2.y;
                } else {
                    pr[0] = p_lds[r];
                }
#pragma unroll
                for (int hh = 0; hh < GQ; hh++) {
                    x0[hh] = __builtin_fmaf(pr[hh], vx, x0[hh]);
                    x1[hh] = __builtin_fmaf(pr[hh], vy, x1[hh]);
                }
            }
        }
#pragma unroll
        for (int hh = 0; hh < GQ; hh++) {
            // merge into the running state (head hh's (m, l) sit in lane hh)
            const float mc = readlane_f(m, hh), lc = readlane_f(ls, hh);
            const float mn = fmaxf(Mr[hh], mc);
            const float fo = __builtin_amdgcn_exp2f(Mr[hh] - mn);
            const float fc = __builtin_amdgcn_exp2f(mc - mn);
            O0[hh] = __builtin_fmaf(O0[hh], fo, x0[hh] * fc);
            O1[hh] = __builtin_fmaf(O1[hh], fo, x1[hh] * fc);
            Lr[hh] = __builtin_fmaf(Lr[hh], fo, lc * fc);
            Mr[hh] = mn;
        }
    }
#pragma unroll
    for (int hh = 0; hh < GQ; hh++) {
        const int64_t pi = ((int64_t)b * a.q_heads + hk * GQ + hh) * a.items + a.splits +
                           a.tail_items + mi;
        *(float2 *)&a.part_o[pi * D + 2 * l] = (float2){O0[hh], O1[hh]};
        if (l == 0) {
            a.part_ml[2 * pi] = Mr[hh];
            a.part_ml[2 * pi + 1] = Lr[hh];
        }
    }
}

template <int BITS, int GQ, bool OUT = false, bool DEEP = false, bool SPLIT = false>
__global__ __launch_bounds__(64) void decode_kernel(DecodeArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t pipe[decode_lds_bytes<BITS, OUT, DEEP>()];
    __shared__ uint4 q_lds[64];
    const int64_t item = blockIdx.x;
    const int64_t streams = (int64_t)a.batch * a.kv_heads;
    if (item < streams * a.tail_items) {
        const int stream = (int)(item % streams), ti = (int)(item / streams);
        if (a.ring_is_f32) decode_tail_f32<GQ>(a, stream, ti);
        else if (a.q_is_f32) decode_tail_f16<GQ, true>(a, stream, ti, pipe);
        else decode_tail_f16<GQ, false>(a, stream, ti, pipe);
        return;
    }
    // paper policy: the items of the groups with partial value codes
    // (a.mixed_items per stream, 0 otherwise), staged in the same LDS
    const int64_t mixed_blocks = streams * a.mixed_items;
    if (item < streams * a.tail_items + mixed_blocks) {
        static_assert(stage_bytes<BITS, OUT>() + GQ * G * 4 + kMixedRowBytes <=
                          decode_lds_bytes<BITS, OUT, DEEP>(),
                      "mixed items stage a block, p and value rows in the ring's LDS");
        const int64_t mt = item - streams * a.tail_items;
        const int stream = (int)(mt % streams), mi = (int)(mt / streams);
        if (a.ring_is_f32) {
            if (a.q_is_f32) decode_mixed_t<BITS, GQ, true, true, OUT, SPLIT>(a, stream, mi, pipe, q_lds);
            else decode_mixed_t<BITS, GQ, true, false, OUT, SPLIT>(a, stream, mi, pipe, q_lds);
        } else {
            if (a.q_is_f32) decode_mixed_t<BITS, GQ, false, true, OUT, SPLIT>(a, stream, mi, pipe, q_lds);
            else decode_mixed_t<BITS, GQ, false, false, OUT, SPLIT>(a, stream, mi, pipe, q_lds);
        }
        return;
    }
    // (q's dtype selects an instantiation: the prologue's loads must not
    // meet at a control-flow join, where the compiler would wait for them)
    // split item it: quarter r, then stream, then split (kQuarterWeight)
    // (in 32 bits: the launch keeps every block number below 2^31)
    const uint32_t it = (uint32_t)(item - streams * a.tail_items - mixed_blocks), st = (uint32_t)streams;
    uint32_t k0 = 0;
    int r = 0;
    for (; r < 3 && it >= st * (k0 + (uint32_t)quarter_splits(a.splits, r)); r++)
        k0 += (uint32_t)quarter_splits(a.splits, r);
    const uint32_t u = (uint32_t)quarter_splits(a.splits, r);
    const uint32_t rem = it - st * k0, sq = rem / u;
    const int stream = (int)sq, sp = (int)(k0 + (rem - sq * u));
    if (a.q_is_f32)
        decode_split<BITS, GQ, true, OUT, DEEP, SPLIT>(a, stream, sp, pipe, q_lds);
    else
        decode_split<BITS, GQ, false, OUT, DEEP, SPLIT>(a, stream, sp, pipe, q_lds);
}

// Merge the partials of one output row (a (batch, query head) of the decode
// step, or a (batch, query head, query) of the attention of T queries):
// part_o [rows][items][D], part_ml [rows][items][2].  The weights 2^(m_s - M)
// are computed once in LDS.  Thread t sums channel t % D over the items
// s = t / D (mod kCombineParts), four loads in flight; the parts are added in
// LDS.  (A row is latency-bound: the parts shorten its chain of loads.)
constexpr int kMaxItems = 4160;
constexpr int kCombineParts = 4;
constexpr int kCombineThreads = D * kCombineParts;

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    return x;
}
__global__ __launch_bounds__(kCombineThreads) void combine_rows_kernel(const float *part_o,
                                                                       const float *part_ml,
                                                                       float *out, int items) {
    constexpr int NW = kCombineThreads / 64;
    __shared__ float w[kMaxItems];
    __shared__ float red[NW];
    __shared__ float acc_s[kCombineThreads];
    const int64_t row = blockIdx.x;
    const int t = threadIdx.x, wv = t >> 6;
    const float *ml = part_ml + row * items * 2;
    float M = -INFINITY;
    for (int s = t; s < items; s += kCombineThreads)
        if (ml[2 * s + 1] > 0.f) M = fmaxf(M, ml[2 * s]);
    M = wave_max(M);
    if ((t & 63) == 0) red[wv] = M;
    __syncthreads();
    M = red[0];
#pragma unroll
    for (int i = 1; i < NW; i++) M = fmaxf(M, red[i]);
    __syncthreads();                            // red is reused below
    float Lp = 0.f;
    for (int s = t; s < items; s += kCombineThreads) {
        const float ls = ml[2 * s + 1];
        const float ws = ls > 0.f ? __builtin_amdgcn_exp2f(ml[2 * s] - M) : 0.f;
        w[s] = ws;
        Lp = __builtin_fmaf(ls, ws, Lp);
    }
    Lp = wave_sum(Lp);
    if ((t & 63) == 0) red[wv] = Lp;
    __syncthreads();                            // w and red are complete
    float L = red[0];
#pragma unroll
    for (int i = 1; i < NW; i++) L += red[i];
    const int c = t % D, part = t / D;
    const float *po = part_o + row * items * D + c;
    float acc0 = 0.f, acc1 = 0.f, acc2 = 0.f, acc3 = 0.f;
    constexpr int P = kCombineParts;
    int s = part;
    for (; s + 3 * P < items; s += 4 * P) {
        acc0 = __builtin_fmaf(po[(int64_t)s * D], w[s], acc0);
        acc1 = __builtin_fmaf(po[(int64_t)(s + P) * D], w[s + P], acc1);
        acc2 = __builtin_fmaf(po[(int64_t)(s + 2 * P) * D], w[s + 2 * P], acc2);
        acc3 = __builtin_fmaf(po[(int64_t)(s + 3 * P) * D], w[s + 3 * P], acc3);
    }
    for (; s < items; s += P) acc0 = __builtin_fmaf(po[(int64_t)s * D], w[s], acc0);
    acc_s[t] = (acc0 + acc1) + (acc2 + acc3);
    __syncthreads();
    if (part == 0) {
        float acc = acc_s[c];
#pragma unroll
        for (int i = 1; i < P; i++) acc += acc_s[c + i * D];
        out[row * D + c] = acc / L;
    }
}

// Rows of at most kFewItems partials: every thread issues all of its loads
// at once (items s = part + kCombineParts * k, its channel t % D of each and
// their (m, l)), so the row costs a single memory round trip; the weights
// 2^(m_s - M) and both sums come from registers, and the parts meet in LDS.
constexpr int kFewPerPart = 16;
constexpr int kFewItems = kCombineParts * kFewPerPart;
__global__ __launch_bounds__(kCombineThreads) void combine_rows_few_kernel(const float *part_o,
                                                                           const float *part_ml,
                                                                           float *out, int items) {
    constexpr int NW = kCombineThreads / 64;
    constexpr int P = kCombineParts;
    __shared__ float red[NW];
    __shared__ float acc_s[kCombineThreads];
    __shared__ float l_s[P];
    const int64_t row = blockIdx.x;
    const int t = threadIdx.x, wv = t >> 6;
    const int c = t % D, part = t / D;          // a wavefront lies within one part
    const float *ml = part_ml + row * items * 2;
    const float *po = part_o + row * items * D + c;
    float o[kFewPerPart], m[kFewPerPart], lw[kFewPerPart];
#pragma unroll
    for (int k = 0; k < kFewPerPart; k++) {
        const int sidx = part + P * k;
        if (sidx < items) {
            o[k] = po[(int64_t)sidx * D];
            const float2 x = *(const float2 *)(ml + 2 * sidx);
            m[k] = x.x;
            lw[k] = x.y;
        } else {
            o[k] = 0.f;
            m[k] = -INFINITY;
            lw[k] = 0.f;
        }
    }
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < kFewPerPart; k++)
        if (lw[k] > 0.f) M = fmaxf(M, m[k]);
    if ((t & 63) == 0) red[wv] = M;
    __syncthreads();
    M = red[0];
#pragma unroll
    for (int i = 1; i < NW; i++) M = fmaxf(M, red[i]);
    float acc = 0.f, L = 0.f;
#pragma unroll
    for (int k = 0; k < kFewPerPart; k++) {
        const float w = lw[k] > 0.f ? __builtin_amdgcn_exp2f(m[k] - M) : 0.f;
        acc = __builtin_fmaf(o[k], w, acc);
        L = __builtin_fmaf(lw[k], w, L);
    }
    acc_s[t] = acc;
    if (c == 0) l_s[part] = L;
    __syncthreads();
    if (part == 0) {
        float a = acc_s[c], Lt = l_s[0];
#pragma unroll
        for (int i = 1; i < P; i++) {
            a += acc_s[c + i * D];
            Lt += l_s[i];
        }
        out[row * D + c] = a / Lt;
    }
}

// Merge `rows` rows of `items` partials each.
static void launch_combine(const float *part_o, const float *part_ml, float *out, int64_t rows,
                           int items, hipStream_t s) {
    if (items <= kFewItems)
        hipLaunchKernelGGL(combine_rows_few_kernel, dim3((unsigned)rows), dim3(kCombineThreads), 0, s,
                           part_o, part_ml, out, items);
    else
        hipLaunchKernelGGL(combine_rows_kernel, dim3((unsigned)rows), dim3(kCombineThreads), 0, s,
                           part_o, part_ml, out, items);
}

// ===========================================================================
// Attention of T queries per (batch, query head) over the packed cache
// ===========================================================================
// The same products as the decode path, with the matrix core's 16 columns
// holding QT = 16 / GQ queries x GQ heads (column j: query j / GQ of the
// wavefront's block, head j % GQ): no column is a replica, so each value
// channel group gets its own B operand.  The wavefronts of a workgroup
// (kAttnColBlocks / CB, CB column blocks each) share each group's block:
// wavefront 0 copies it HBM -> LDS and one barrier per two groups hands it to
// all.  p is kept as P_s = 2^(s - m - kSlack)
// in fp16 (<= 1); the sums of p and of p * vzero run on the matrix core, and
// every accumulator carries the same 2^-kSlack, which cancels in o = acc / l.

// Online-softmax step over the 8 scores a lane holds.  nm caches -m_run -
// kSlack.  Returns P_s as fp16 pairs in operand order.
__device__ __forceinline__ void attn_softmax(f4 &S0, f4 &S1, float cs, float kbl, float &m_run,
                                             float &m_thr, float &nm, f4 &Lsum, f4 &Vz,
                                             f4 (&accV)[8], h2 (&Ps)[4]) {
    float mt = vmax(vmax(vmax(S0[0], S0[1]), vmax(S0[2], S0[3])),
                    vmax(vmax(S1[0], S1[1]), vmax(S1[2], S1[3])));
    mt = __builtin_fmaf(mt, cs, kbl);
    if (__any(mt > m_thr)) {
        const float m_new = vmax(m_run, xmax_rows(mt));
        const float al = __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
        for (int o = 0; o < 8; o++) accV[o] *= al;
        Lsum *= al;
        Vz *= al;
        nm = -m_new - (float)kSlack;
        m_run = m_new;
        m_thr = m_new + (float)kSlack;
    }
    const float nk = nm + kbl;
    float p[8];
#pragma unroll
    for (int e = 0; e < 4; e++) {
        p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(S0[e], cs, nk));
        p[4 + e] = __builtin_amdgcn_exp2f(__builtin_fmaf(S1[e], cs, nk));
    }
#pragma unroll
    for (int m = 0; m < 4; m++) {
        Ps[m][0] = (_Float16)p[2 * m];
        Ps[m][1] = (_Float16)p[2 * m + 1];
    }
}

// Scores of rows past `last_ok` (and, causally, of tokens past the lane's
// query) become -inf.  Row r of tile t is token tok0 + 16t + 4Gl + e.
__device__ __forceinline__ void mask_scores(f4 &S0, f4 &S1, int64_t tok0, int Gl, int cnt,
                                            int64_t pq) {
#pragma unroll
    for (int e = 0; e < 4; e++) {
        const int r0 = 4 * Gl + e, r1 = 16 + 4 * Gl + e;
        if (r0 >= cnt || tok0 + r0 > pq) S0[e] = -INFINITY;
        if (r1 >= cnt || tok0 + r1 > pq) S1[e] = -INFINITY;
    }
}

template <int BITS, int GQ, bool QF32, int CB, bool OUT = false, bool SPLIT = false>
__global__ __launch_bounds__(64 * (kAttnColBlocks / CB), BITS == 2 ? (CB == 1 ? 4 : 2) : 1)
void attn_kernel(AttnArgs a) {
    using PP = Pipe<BITS>;
    constexpr int W = kAttnColBlocks / CB;      // wavefronts
    constexpr int QT = 16 / GQ;                 // queries per column block
    constexpr int DPL = 2 * BITS;
    constexpr int VTS = 40;                     // fp16 per transposed value row (80 B)
    constexpr int SB = stage_bytes<BITS, OUT>();   // block (+ outlier record)
    // ring stages: the wavefronts meet at one barrier per two groups, with up
    // to four groups in flight at 2 bits (two at 4 and 8 bits)
    constexpr int AST = BITS == 2 ? 6 : 4;
    __shared__ __attribute__((aligned(16))) uint8_t ring[AST * SB];
    __shared__ uint4 qs[W][CB][4][64];          // unscaled fp16 q, B-operand order
    __shared__ __attribute__((aligned(16))) _Float16 vt[D * VTS];

    const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int j = l & 15, Gl = l >> 4;
    const int h = j % GQ;
    const int split = (int)(blockIdx.x % (unsigned)a.splits);
    const int64_t sq = blockIdx.x / (unsigned)a.splits;
    const int qb = (int)(sq % a.qblocks);
    const int stream = (int)(sq / a.qblocks);
    const int b = stream / a.kv_heads, hk = stream % a.kv_heads;
    const int64_t T = a.T, n = a.n_tokens;
    // column block c of this wavefront: queries qi0[c] .. qi0[c] + QT - 1
    const int64_t qw0 = ((int64_t)qb * W + w) * CB * QT;
    const bool wave_ok = qw0 < T;
    const int64_t pq_wave = a.causal ? n - T + qw0 : n - 1;   // smallest in the wave
    int64_t qi_wg = ((int64_t)qb + 1) * W * CB * QT - 1;
    if (qi_wg > T - 1) qi_wg = T - 1;
    const int64_t pq_wg = a.causal ? n - T + qi_wg : n - 1;
    int64_t qi[CB], pq[CB];
    bool col_ok[CB];
#pragma unroll
    for (int c = 0; c < CB; c++) {
        qi[c] = qw0 + c * QT + j / GQ;
        col_ok[c] = qi[c] < T;
        pq[c] = a.causal ? n - T + qi[c] : n - 1;             // last token the column sees
    }

    // groups with key and value codes: [0, ngv); under the paper policy the
    // groups [ngv, ng) have key codes and value codes below n_vquant only
    const int64_t ng = a.n_quant / G;
    const int64_t ngv = (a.n_vquant < a.n_quant ? a.n_vquant : a.n_quant) / G;
    const int64_t g0 = (int64_t)split * a.groups_per_split;
    int64_t g1 = g0 + a.groups_per_split < ngv ? g0 + a.groups_per_split : ngv;
    if (g1 > pq_wg / G + 1) g1 = pq_wg / G + 1;        // groups past every query
    const int n_g = g1 > g0 ? (int)(g1 - g0) : 0;

    const uint8_t *sblk = a.blocks + ((int64_t)stream * a.max_groups + g0) * a.block_bytes;
    const uint8_t *srec = OUT ? a.outliers + ((int64_t)stream * a.max_groups + g0) * kOutlierRecordBytes
                              : nullptr;
    const int64_t bstride = SPLIT ? a.block_bytes : PP::BB;
    // split layout: key unit of group gi, value slots (cg >> vsh of nvs)
    const uint8_t *skside = a.side.kside + (int64_t)stream * a.side.max_kunits * (4 * D);
    auto kunit = [&](int64_t gi) { return skside + (gi >> a.side.kunit_shift) * (4 * D); };
    const int vsh = SPLIT ? a.side.vsh : 0, nvs = SPLIT ? a.side.nvs : 4;
    const uint32_t rbase = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void *)ring;
    h2 qB[CB][4][4];
#pragma unroll
    for (int c = 0; c < CB; c++) {
        const int64_t qrow =
            (((int64_t)b * a.q_heads + hk * GQ + h) * T + (col_ok[c] ? qi[c] : 0)) * D;
        load_q_operand<QF32>(a.q, qrow, Gl, qB[c]);
    }
    int issued = 0, is = 0, rs = 0;
    if (w == 0) {
        for (; issued < AST - 2 && issued < n_g; issued++) {
            issue_group<BITS, OUT, SPLIT>(sblk + (int64_t)issued * bstride,
                                          OUT ? srec + (int64_t)issued * kOutlierRecordBytes : nullptr,
                                          rbase + (uint32_t)is * SB, l, false,
                                          SPLIT ? kunit(g0 + issued) : nullptr, 32 * nvs);
            is = is + 1 == AST ? 0 : is + 1;
        }
    }
#pragma unroll
    for (int c = 0; c < CB; c++) {
#pragma unroll
        for (int s = 0; s < 4; s++)
#pragma unroll
            for (int m = 0; m < 4; m++) {
                asm volatile("" : "+v"(qB[c][s][m]));
                if (!col_ok[c]) qB[c][s][m] = (h2){(_Float16)0.f, (_Float16)0.f};
            }
#pragma unroll
        for (int s = 0; s < 4; s++) {
            uint4 u;
            u.x = __builtin_bit_cast(uint32_t, qB[c][s][0]);
            u.y = __builtin_bit_cast(uint32_t, qB[c][s][1]);
            u.z = __builtin_bit_cast(uint32_t, qB[c][s][2]);
            u.w = __builtin_bit_cast(uint32_t, qB[c][s][3]);
            qs[w][c][s][l] = u;
        }
#pragma unroll
        for (int m = 0; m < 4; m++) {
            const _Float16 dn = (_Float16)(1.0f / (float)(1 << kScaleLog2<BITS>(m)));
            const h2 d2 = {dn, dn};
#pragma unroll
            for (int s = 0; s < 4; s++) qB[c][s][m] = qB[c][s][m] * d2;
        }
    }
    h8 ones;
#pragma unroll
    for (int i = 0; i < 8; i++) ones[i] = (_Float16)1.0f;

    float m_run[CB], m_thr[CB], nm[CB];
    f4 Lsum[CB], Vz[CB], accV[CB][8];
#pragma unroll
    for (int c = 0; c < CB; c++) {
        m_run[c] = -INFINITY;
        m_thr[c] = -INFINITY;
        nm[c] = 0.f;
        Lsum[c] = (f4){0.f, 0.f, 0.f, 0.f};
        Vz[c] = Lsum[c];
#pragma unroll
        for (int o = 0; o < 8; o++) accV[c][o] = (f4){0.f, 0.f, 0.f, 0.f};
    }
    const float csq = a.sm_log2 * kTwo24;

    // Scores of the 32 tokens of the block at stg against every column:
    // key-zero bias (every row of a column holds it), the code products (each
    // key operand unpacked once for all column blocks) and, with outlier-aware
    // keys, q . K over the kept channels.  Units of 2^-24 (csq converts).
    auto block_scores = [&](const uint8_t *stg, f4 (&Sk)[CB], f4 (&S0)[CB], f4 (&S1)[CB]) {
        const uint4 *side = (const uint4 *)(stg + 2 * PP::CB);
        uint32_t kc[DPL];
#pragma unroll
        for (int w4 = 0; w4 < BITS / 2; w4++) {
            const uint4 u = *(const uint4 *)(stg + w4 * 1024 + 16 * l);
            kc[4 * w4] = u.x; kc[4 * w4 + 1] = u.y; kc[4 * w4 + 2] = u.z; kc[4 * w4 + 3] = u.w;
        }
#pragma unroll
        for (int c = 0; c < CB; c++) {
            Sk[c] = (f4){0.f, 0.f, 0.f, 0.f};
            S0[c] = Sk[c];
            S1[c] = Sk[c];
        }
#pragma unroll
        for (int s = 0; s < 4; s++) {
            const h8 kz = __builtin_bit_cast(h8, side[16 + 4 * s + Gl]);
#pragma unroll
            for (int c = 0; c < CB; c++)
                Sk[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                    kz, __builtin_bit_cast(h8, qs[w][c][s][l]), Sk[c], 0, 0, 0);
        }
#pragma unroll
        for (int s = 0; s < 4; s++) {
            h2 ks[4];
            split4(side[4 * s + Gl], ks);
            const h8 A0 = unpack_operand<BITS>(kc, s), A1 = unpack_operand<BITS>(kc, 4 + s);
#pragma unroll
            for (int c = 0; c < CB; c++) {
                h2 qh[4], ql[4];
#pragma unroll
                for (int m = 0; m < 4; m++) {
                    qh[m] = qB[c][s][m] * ks[m];
                    ql[m] = __builtin_elementwise_fma(qB[c][s][m], ks[m], -qh[m]);
                }
                const h8 Bh = pack_h8(qh), Bl = pack_h8(ql);
                S0[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A0, Bh, S0[c], 0, 0, 0);
                S1[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A1, Bh, S1[c], 0, 0, 0);
                S0[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A0, Bl, S0[c], 0, 0, 0);
                S1[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A1, Bl, S1[c], 0, 0, 0);
            }
        }
        if constexpr (OUT) {
            // key channels kept in fp16 (codes, scale and zero 0): add q . K
            // over them from the record, in the scores' units of 2^24.  q of
            // column j at channel ch sits in the unscaled B operand of step
            // ch / 32, lane j + 16 ((ch % 32) / 8), element ch % 8.
            const uint2 idx = *(const uint2 *)(stg + PP::BB);
            const int ch[kMaxKeyOutliers] = {(int)(idx.x & 0xFFFFu), (int)(idx.x >> 16),
                                             (int)(idx.y & 0xFFFFu)};
            const _Float16 *rval = (const _Float16 *)(stg + PP::BB + 16);
#pragma unroll
            for (int o = 0; o < kMaxKeyOutliers; o++) {
                if (o < a.n_out) {
                    const int co = ch[o];
                    const int qe = ((co >> 5) * 64 + j + 16 * ((co >> 3) & 3)) * 8 + (co & 7);
                    const h2 *v0 = (const h2 *)(rval + G * o + 4 * Gl);
                    const h2 *v1 = (const h2 *)(rval + G * o + 16 + 4 * Gl);
#pragma unroll
                    for (int c = 0; c < CB; c++) {
                        const float qo = (float)((const _Float16 *)&qs[w][c][0][0])[qe] * kTwoM24;
#pragma unroll
                        for (int e = 0; e < 4; e++) {
                            S0[c][e] = __builtin_fmaf(qo, (float)v0[e >> 1][e & 1], S0[c][e]);
                            S1[c][e] = __builtin_fmaf(qo, (float)v1[e >> 1][e & 1], S1[c][e]);
                        }
                    }
                }
            }
        }
    };

    for (int g = 0; g < n_g; g++) {
        if ((g & 1) == 0) {
            // groups g and g + 1 landed; every wave is done with g - 1, so the
            // stages up to group g - 1 + AST are free
            const int last = g + 1 < n_g ? g + 1 : g;
            if (w == 0) {
                constexpr int P = SPLIT ? 2 * Pipe<BITS>::CB / 1024 + 3 : Pipe<BITS>::DPG + (OUT ? 1 : 0);
                const int r = issued - 1 - last;
                if (r >= 4) wait_vm<4 * P>();
                else if (r == 3) wait_vm<3 * P>();
                else if (r == 2) wait_vm<2 * P>();
                else if (r == 1) wait_vm<P>();
                else wait_vm<0>();
            }
            __syncthreads();
            if (w == 0) {
                for (; issued < n_g && issued <= g + AST - 1; issued++) {
                    issue_group<BITS, OUT, SPLIT>(
                        sblk + (int64_t)issued * bstride,
                        OUT ? srec + (int64_t)issued * kOutlierRecordBytes : nullptr,
                        rbase + (uint32_t)is * SB, l, false, SPLIT ? kunit(g0 + issued) : nullptr,
                        32 * nvs);
                    is = is + 1 == AST ? 0 : is + 1;
                }
            }
        }
        const uint8_t *stg = ring + rs * SB;
        rs = rs + 1 == AST ? 0 : rs + 1;
        if (!wave_ok) continue;
        const uint4 *side = (const uint4 *)(stg + 2 * PP::CB);
        const uint2 *s2 = (const uint2 *)side;
        uint32_t vc[DPL];
#pragma unroll
        for (int w4 = 0; w4 < BITS / 2; w4++) {
            const uint4 v = *(const uint4 *)(stg + PP::CB + w4 * 1024 + 16 * l);
            vc[4 * w4] = v.x; vc[4 * w4 + 1] = v.y; vc[4 * w4 + 2] = v.z; vc[4 * w4 + 3] = v.w;
        }
        f4 Sk[CB], S0[CB], S1[CB];
        block_scores(stg, Sk, S0, S1);
        const int64_t tok0 = (g0 + g) * G;
        const bool masked = tok0 + G - 1 > pq_wave;
        h2 Pc[CB][4];
        const int cz = j & 3;
        const int zi = 64 + 8 * nvs + 8 * (cz >> vsh) + Gl;
        const uint2 z0 = s2[zi], z1 = s2[zi + 4];
        const uint4 zz = {z0.x, z0.y, z1.x, z1.y};
#pragma unroll
        for (int c = 0; c < CB; c++) {
            if (masked) mask_scores(S0[c], S1[c], tok0, Gl, G, pq[c]);
            h2 Ps[4];
            attn_softmax(S0[c], S1[c], csq, Sk[c][0] * a.sm_log2, m_run[c], m_thr[c], nm[c],
                         Lsum[c], Vz[c], accV[c], Ps);
            const h8 Bp = pack_h8(Ps);
            Lsum[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, Bp, Lsum[c], 0, 0, 0);
            // value-zero bias: A row r carries vzero of channel group r % 4
            Vz[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, zz), Bp, Vz[c],
                                                          0, 0, 0);
#pragma unroll
            for (int m = 0; m < 4; m++) {
                const _Float16 dn = (_Float16)(1.0f / (float)(1 << kScaleLog2<BITS>(m)));
                Pc[c][m] = m == 0 ? Ps[m] : Ps[m] * (h2){dn, dn};
            }
        }
#pragma unroll
        for (int cg = 0; cg < 4; cg++) {
            const int si = 64 + 8 * (cg >> vsh) + Gl;
            const uint2 a0 = s2[si], a1 = s2[si + 4];
            const h2 v0 = __builtin_bit_cast(h2, a0.x), v1 = __builtin_bit_cast(h2, a0.y);
            const h2 v2 = __builtin_bit_cast(h2, a1.x), v3 = __builtin_bit_cast(h2, a1.y);
            const h8 U0 = unpack_operand<BITS>(vc, 2 * cg), U1 = unpack_operand<BITS>(vc, 2 * cg + 1);
#pragma unroll
            for (int c = 0; c < CB; c++) {
                h2 ps[4];
                ps[0] = Pc[c][0] * v0;
                ps[1] = Pc[c][1] * v1;
                ps[2] = Pc[c][2] * v2;
                ps[3] = Pc[c][3] * v3;
                const h8 Bv = pack_h8(ps);
                accV[c][2 * cg] = __builtin_amdgcn_mfma_f32_16x16x32_f16(U0, Bv, accV[c][2 * cg],
                                                                        0, 0, 0);
                accV[c][2 * cg + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                    U1, Bv, accV[c][2 * cg + 1], 0, 0, 0);
            }
        }
    }
    // code products carry 2^-24: bring them to the residual's units
#pragma unroll
    for (int c = 0; c < CB; c++)
#pragma unroll
        for (int o = 0; o < 8; o++) accV[c][o] *= kTwo24;

    // Paper policy: the last split walks the groups [ngv, ng), whose keys are
    // codes but whose values are codes only below n_vquant (in the first of
    // them; at most 31 tokens) and ring rows from there on.  Per group the
    // workgroup copies the block into ring stage 0 and stages the 32 value
    // rows transposed in LDS, the coded ones as fp16 of code * scale + zero
    // (float32, two roundings, then one to fp16); each wavefront computes the
    // scores from the key codes as in the loop above and p . V from LDS as in
    // the residual below.
    if (split == a.splits - 1 && ng > ngv) {
        constexpr uint32_t M1 = (1u << BITS) - 1u;
        const _Float16 *rvh = (const _Float16 *)a.ring_v + (int64_t)stream * a.ring_cap * D;
        const float *rvf = (const float *)a.ring_v + (int64_t)stream * a.ring_cap * D;
        for (int64_t gm = ngv; gm < ng && gm * G <= pq_wg; gm++) {
            const int64_t tok0 = gm * G;
            __syncthreads();        // stage 0 and the transposed rows are free
            const uint4 *blk =
                (const uint4 *)(a.blocks + ((int64_t)stream * a.max_groups + gm) * a.block_bytes);
            if constexpr (SPLIT) {
                // codes, the key unit where a G = 32 block has its key scale
                // and zero, then the value pairs
                const uint4 *ku = (const uint4 *)kunit(gm);
                constexpr int C16 = 2 * PP::CB / 16;
                for (int i = threadIdx.x; i < C16 + 32 + 8 * nvs; i += 64 * W)
                    ((uint4 *)ring)[i] = i < C16 ? blk[i] : i < C16 + 32 ? ku[i - C16] : blk[i - 32];
            } else {
                for (int i = threadIdx.x; i < PP::BB / 16; i += 64 * W) ((uint4 *)ring)[i] = blk[i];
            }
            if constexpr (OUT) {
                const uint4 *rec = (const uint4 *)(a.outliers + ((int64_t)stream * a.max_groups + gm) *
                                                                    kOutlierRecordBytes);
                if (threadIdx.x < kOutlierRecordBytes / 16)
                    ((uint4 *)(ring + PP::BB))[threadIdx.x] = rec[threadIdx.x];
            }
            __syncthreads();
            {
#pragma clang fp contract(off)
                const uint32_t *vcode = (const uint32_t *)(ring + PP::CB);
                const _Float16 *sd = (const _Float16 *)(ring + 2 * PP::CB);
                // the group's rows wrap around the ring (more than G slots) at most once
                const int64_t slot0 = tok0 % a.ring_cap;
                for (int idx = threadIdx.x; idx < G * D; idx += 64 * W) {
                    const int r = idx / D, c = idx % D;
                    const int64_t t = tok0 + r;
                    _Float16 v;
                    if (t < a.n_vquant) {
                        int dw, bit;
                        code_pos<BITS>(true, r, c, dw, bit);
                        const float vs = (float)sd[2 * D + G * ((c / G) >> vsh) + r];
                        const float vz = (float)sd[2 * D + G * (nvs + ((c / G) >> vsh)) + r];
                        v = (_Float16)((float)((vcode[dw] >> bit) & M1) * vs + vz);
                    } else {
                        const int64_t sl = slot0 + r < a.ring_cap ? slot0 + r : slot0 + r - a.ring_cap;
                        const int64_t ri = sl * D + c;
                        v = a.ring_f32 ? (_Float16)rvf[ri] : rvh[ri];
                    }
                    vt[c * VTS + r] = v;
                }
            }
            __syncthreads();
            if (!wave_ok) continue;
            f4 Sk[CB], S0[CB], S1[CB];
            block_scores(ring, Sk, S0, S1);
            h8 Bp[CB];
#pragma unroll
            for (int c = 0; c < CB; c++) {
                if (tok0 + G - 1 > pq_wave) mask_scores(S0[c], S1[c], tok0, Gl, G, pq[c]);
                h2 Ps[4];
                attn_softmax(S0[c], S1[c], csq, Sk[c][0] * a.sm_log2, m_run[c], m_thr[c], nm[c],
                             Lsum[c], Vz[c], accV[c], Ps);
                Bp[c] = pack_h8(Ps);
                Lsum[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, Bp[c], Lsum[c], 0, 0, 0);
            }
#pragma unroll
            for (int o = 0; o < 8; o++) {
                const _Float16 *row = vt + (16 * o + j) * VTS;
                const uint2 v0 = *(const uint2 *)(row + 4 * Gl);
                const uint2 v1 = *(const uint2 *)(row + 16 + 4 * Gl);
                const uint4 vv = {v0.x, v0.y, v1.x, v1.y};
#pragma unroll
                for (int c = 0; c < CB; c++)
                    accV[c][o] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, vv),
                                                                       Bp[c], accV[c][o], 0, 0, 0);
            }
        }
    }

    // The last split walks the residual [Q, n) in 32-token chunks: the
    // workgroup stages the chunk's value rows transposed in LDS (channel
    // rows), each wavefront reads its K rows straight from the ring.  Rows
    // of a float32 ring enter the fp16 products rounded to nearest fp16.
    if (split == a.splits - 1 && n > a.n_quant) {
        const int64_t nres = n - a.n_quant;
        const int cap = (int)a.ring_cap;
        const int rb = a.ring_f32 ? 4 : 2;              // bytes per ring element
        const char *rkb = (const char *)a.ring_k + (int64_t)stream * a.ring_cap * D * rb;
        const char *rvb = (const char *)a.ring_v + (int64_t)stream * a.ring_cap * D * rb;
        const int slot_q = (int)(a.n_quant % a.ring_cap);
        for (int64_t c0 = 0; c0 < nres && a.n_quant + c0 <= pq_wg; c0 += G) {
            const int cnt = nres - c0 < G ? (int)(nres - c0) : G;
            auto slot = [&](int r) {
                int s3 = slot_q + (int)(c0 % a.ring_cap) + (r < cnt ? r : cnt - 1);
                while (s3 >= cap) s3 -= cap;
                return s3;
            };
            __syncthreads();        // the previous chunk's transposed rows are read
            for (int idx = threadIdx.x; idx < G * (D / 8); idx += 64 * W) {
                const int r = idx >> 4, piece = idx & 15;
                const char *src = rvb + ((int64_t)slot(r) * D + 8 * piece) * rb;
                h2 hv[4];
                if (a.ring_f32) {
                    const float4 x0 = *(const float4 *)src, x1 = *(const float4 *)(src + 16);
                    hv[0] = (h2){(_Float16)x0.x, (_Float16)x0.y};
                    hv[1] = (h2){(_Float16)x0.z, (_Float16)x0.w};
                    hv[2] = (h2){(_Float16)x1.x, (_Float16)x1.y};
                    hv[3] = (h2){(_Float16)x1.z, (_Float16)x1.w};
                } else {
                    split4(*(const uint4 *)src, hv);
                }
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    vt[(8 * piece + 2 * i) * VTS + r] = hv[i][0];
                    vt[(8 * piece + 2 * i + 1) * VTS + r] = hv[i][1];
                }
            }
            __syncthreads();
            if (!wave_ok) continue;
            f4 S[CB][2];
#pragma unroll
            for (int c = 0; c < CB; c++) S[c][0] = S[c][1] = (f4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int t = 0; t < 2; t++) {
                // lane (j, Gl) takes channels 32s + 8Gl .. + 7 of row 16t + j
                const char *krow = rkb + ((int64_t)slot(16 * t + j) * D + 8 * Gl) * rb;
#pragma unroll
                for (int s = 0; s < 4; s++) {
                    h8 kk;
                    if (a.ring_f32) {
                        const float4 x0 = *(const float4 *)(krow + 128 * s);
                        const float4 x1 = *(const float4 *)(krow + 128 * s + 16);
                        kk = (h8){(_Float16)x0.x, (_Float16)x0.y, (_Float16)x0.z, (_Float16)x0.w,
                                  (_Float16)x1.x, (_Float16)x1.y, (_Float16)x1.z, (_Float16)x1.w};
                    } else {
                        kk = __builtin_bit_cast(h8, *(const uint4 *)(krow + 64 * s));
                    }
#pragma unroll
                    for (int c = 0; c < CB; c++)
                        S[c][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                            kk, __builtin_bit_cast(h8, qs[w][c][s][l]), S[c][t], 0, 0, 0);
                }
            }
            h8 Bp[CB];
#pragma unroll
            for (int c = 0; c < CB; c++) {
                mask_scores(S[c][0], S[c][1], a.n_quant + c0, Gl, cnt, pq[c]);
                h2 Ps[4];
                attn_softmax(S[c][0], S[c][1], a.sm_log2, 0.f, m_run[c], m_thr[c], nm[c], Lsum[c],
                             Vz[c], accV[c], Ps);
                Bp[c] = pack_h8(Ps);
                Lsum[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, Bp[c], Lsum[c], 0, 0, 0);
            }
#pragma unroll
            for (int o = 0; o < 8; o++) {
                const _Float16 *row = vt + (16 * o + j) * VTS;
                const uint2 v0 = *(const uint2 *)(row + 4 * Gl);
                const uint2 v1 = *(const uint2 *)(row + 16 + 4 * Gl);
                const uint4 vv = {v0.x, v0.y, v1.x, v1.y};
#pragma unroll
                for (int c = 0; c < CB; c++)
                    accV[c][o] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, vv),
                                                                       Bp[c], accV[c][o], 0, 0, 0);
            }
        }
    }

    if (!wave_ok) return;
    // lane (j, Gl) holds channels 16o + 4Gl + e of its column; Vz[e] is the
    // bias of channel group e (rows repeat with period 4)
#pragma unroll
    for (int c = 0; c < CB; c++) {
        if (!col_ok[c]) continue;
        const int64_t row = ((int64_t)b * a.q_heads + hk * GQ + h) * T + qi[c];
        const float L = Lsum[c][0];
        if (a.splits == 1) {
            const float inv = 1.0f / L;
#pragma unroll
            for (int o = 0; o < 8; o++) {
                const float bz = Vz[c][o / 2];
                float4 v;
                v.x = (accV[c][o][0] + bz) * inv;
                v.y = (accV[c][o][1] + bz) * inv;
                v.z = (accV[c][o][2] + bz) * inv;
                v.w = (accV[c][o][3] + bz) * inv;
                *(float4 *)&a.out[row * D + 16 * o + 4 * Gl] = v;
            }
        } else {
            const int64_t pi = row * a.splits + split;
#pragma unroll
            for (int o = 0; o < 8; o++) {
                const float bz = Vz[c][o / 2];
                const float4 v = {accV[c][o][0] + bz, accV[c][o][1] + bz, accV[c][o][2] + bz,
                                  accV[c][o][3] + bz};
                *(float4 *)&a.part_o[pi * D + 16 * o + 4 * Gl] = v;
            }
            if (Gl == 0) {
                a.part_ml[2 * pi] = m_run[c];
                a.part_ml[2 * pi + 1] = L;
            }
        }
    }
}

// ===========================================================================
// Fixed scratch of kivi_decode_attn_noalloc: the decode partials live in a
// file-scope device array instead of a caller workspace, for callers that
// cannot allocate.  Each device holds its own copy until the process ends.
// Host code never passes `scratch` itself to a kernel (on the host the name
// stands for a host-side placeholder): its device address is looked up once
// per device, with that device current, and kept.
// ===========================================================================
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
static std::atomic<void *> g_scratch_ptr[kMaxDevices];

hipError_t noalloc_scratch(void **ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
    *ptr = p;
    return hipSuccess;
}

// ===========================================================================
// Launchers
// ===========================================================================
// Workgroups of kRingThreads pieces that copy a ring append's rows.
static int64_t ring_blocks(const RingArgs &a) {
    const int64_t ntok = a.tok_end - a.tok_begin;
    if (ntok <= 0) return 0;
    const int64_t pieces = (int64_t)a.streams * ntok * (2 * D * a.esize / 16);
    return (pieces + kRingThreads - 1) / kRingThreads;
}

template <int BITS, typename T, int GT, bool OUT = false, bool KSEG = false>
static hipError_t launch_quantize_t(const QuantizeArgs &a, hipStream_t s) {
    // tasks per launched block range: key groups of GT blocks and / or blocks
    // (segment pairs: two per block)
    auto tasks_of = [&](int64_t nb) {
        return KSEG ? 2 * nb : a.kinds == 3 ? nb / GT * (1 + GT) : a.kinds == 1 ? nb / GT : nb;
    };
    const int64_t align = (a.kinds == 2 || KSEG) ? 1 : GT;
    // Blocks with tokens before n_old read rows from the ring; so does a block
    // whose value rows stop at v_limit (only that instance checks the limit).
    int64_t ring_end = (a.n_old + G - 1) / G;
    if (a.kinds != 1 && a.v_limit < a.block_end * G) ring_end = a.block_end;
    int64_t split = ring_end < a.block_begin ? a.block_begin : ring_end;
    split = a.block_begin + (split - a.block_begin + align - 1) / align * align;
    if (split > a.block_end) split = a.block_end;
    // The ring copy (a.copy) rides on the instance that reads no ring row.
    // When every block reads the ring, it rides on that instance instead if
    // none of the slots it writes holds a row the instance reads: the rows
    // read lie in [block_begin * G, n_old) and the rows written below
    // copy.tok_end, so that holds when the two ranges span less than the ring.
    const bool copy = a.copy.tok_end > a.copy.tok_begin;
    const bool ring_carries = copy && a.block_end <= split &&
                              a.copy.tok_end - 1 - a.block_begin * G < a.ring_cap;
    if (split > a.block_begin) {
        QuantizeArgs r = a;
        r.block_end = split;
        const int64_t tasks = (int64_t)a.streams * tasks_of(split - a.block_begin);
        r.quant_tasks = (uint32_t)tasks;
        hipLaunchKernelGGL((quantize_kernel<BITS, T, true, GT, OUT, KSEG>),
                           dim3((unsigned)(tasks + (ring_carries ? ring_blocks(a.copy) : 0))), dim3(64),
                           0, s, r);
    }
    if (a.block_end > split) {
        QuantizeArgs n = a;
        n.block_begin = split;
        const int64_t tasks = (int64_t)a.streams * tasks_of(a.block_end - split);
        n.quant_tasks = (uint32_t)tasks;
        hipLaunchKernelGGL((quantize_kernel<BITS, T, false, GT, OUT, KSEG>),
                           dim3((unsigned)(tasks + ring_blocks(a.copy))), dim3(64), 0, s, n);
        return hipGetLastError();
    }
    // every quantized block reads the ring: unless it rode along, the copy
    // runs after them
    const hipError_t e = hipGetLastError();
    return e != hipSuccess || ring_carries ? e : launch_ring_append(a.copy, s);
}

template <int BITS, typename T>
static hipError_t launch_quantize_g(const QuantizeArgs &a, hipStream_t s) {
    if (a.kinds == 4) return launch_quantize_t<BITS, T, 4, false, true>(a, s);
    if (a.n_out > 0) return launch_quantize_t<BITS, T, 1, true>(a, s);
    if (a.gt == 1) return launch_quantize_t<BITS, T, 1>(a, s);
    if (a.gt == 2) return launch_quantize_t<BITS, T, 2>(a, s);
    return launch_quantize_t<BITS, T, 4>(a, s);
}

hipError_t launch_quantize(const QuantizeArgs &a, hipStream_t s) {
    const bool copy = a.copy.tok_end > a.copy.tok_begin;
    if (copy && a.copy.esize != 2 && a.copy.esize != 4) return hipErrorInvalidValue;
    if (copy && ring_blocks(a.copy) > 0x7FFFFFFF - 2 * (int64_t)a.streams * a.max_groups)
        return hipErrorInvalidValue;
    if (a.block_end <= a.block_begin || a.streams <= 0) return launch_ring_append(a.copy, s);
    if (a.kinds < 1 || a.kinds > 4) return hipErrorInvalidValue;
    // segment pairs: value groups of 128 channels, statistics from seg_stats
    if (a.kinds == 4 && (a.gt != 4 || a.n_out != 0 || !a.seg_stats)) return hipErrorInvalidValue;
    if (a.gt != 1 && a.gt != 2 && a.gt != 4) return hipErrorInvalidValue;
    if (a.n_out < 0 || a.n_out > kMaxKeyOutliers || (a.n_out > 0 && (a.gt != 1 || !a.outliers)))
        return hipErrorInvalidValue;
    // key tasks cover whole groups of gt blocks
    if (a.kinds != 2 && a.kinds != 4 && (a.block_begin % a.gt != 0 || a.block_end % a.gt != 0))
        return hipErrorInvalidValue;
    // every value row the kernel reads must exist: rows >= v_limit are skipped,
    // and only the last block may stop early
    if (a.kinds != 1 && a.v_limit < a.block_end * G && a.v_limit <= (a.block_end - 1) * G)
        return hipErrorInvalidValue;
    if ((int64_t)a.streams * (a.block_end - a.block_begin) * 2 > 0x7FFFFFFF) return hipErrorInvalidValue;
    if (a.bits == 2) return a.is_f32 ? launch_quantize_g<2, float>(a, s) : launch_quantize_g<2, _Float16>(a, s);
    if (a.bits == 8) return a.is_f32 ? launch_quantize_g<8, float>(a, s) : launch_quantize_g<8, _Float16>(a, s);
    return a.is_f32 ? launch_quantize_g<4, float>(a, s) : launch_quantize_g<4, _Float16>(a, s);
}

hipError_t launch_segment_stats(const QuantizeArgs &a, hipStream_t s) {
    const int64_t nb = a.block_end - a.block_begin;
    if (nb <= 0 || a.streams <= 0) return hipSuccess;
    if (!a.seg_stats || !a.seg_partial || a.seg_chunk_blocks < 1 ||
        (int64_t)a.seg_chunks * a.seg_chunk_blocks < nb ||
        (int64_t)(a.seg_chunks - 1) * a.seg_chunk_blocks >= nb)
        return hipErrorInvalidValue;
    const int64_t tasks = (int64_t)a.streams * a.seg_chunks;
    if (tasks > 0x7FFFFFFF) return hipErrorInvalidValue;
    if (a.is_f32)
        hipLaunchKernelGGL(seg_stats_kernel<float>, dim3((unsigned)tasks), dim3(64), 0, s, a);
    else
        hipLaunchKernelGGL(seg_stats_kernel<_Float16>, dim3((unsigned)tasks), dim3(64), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(seg_reduce_kernel, dim3((unsigned)a.streams), dim3(64), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_ring_append(const RingArgs &a, hipStream_t s) {
    if (a.tok_end <= a.tok_begin) return hipSuccess;
    if (a.esize != 2 && a.esize != 4) return hipErrorInvalidValue;
    const int64_t blocks = ring_blocks(a);
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL(ring_append_kernel, dim3((unsigned)blocks), dim3(kRingThreads), 0, s, a);
    return hipGetLastError();
}

// The layouts the kernels read: G = 32 (four value slots, no shift) or the
// split layout (1 or 2 value slots per token, unit shift 0..2, no outlier
// records).
static bool side_args_ok(const SideArgs &sa, int n_out) {
    if (!sa.split) return sa.vsh == 0 && sa.nvs == 4;
    return n_out == 0 && sa.kside && (sa.nvs == 1 || sa.nvs == 2) && sa.vsh >= 1 && sa.vsh <= 2 &&
           (4 >> sa.vsh) == sa.nvs && sa.kunit_shift >= 0 && sa.kunit_shift <= 2;
}

template <int BITS, bool OUT = false, bool DEEP = false, bool SPLIT = false>
static void launch_decode_bits(const DecodeArgs &a, int gq, dim3 grid, hipStream_t s) {
    if (gq == 4) hipLaunchKernelGGL((decode_kernel<BITS, 4, OUT, DEEP, SPLIT>), grid, dim3(64), 0, s, a);
    else if (gq == 2) hipLaunchKernelGGL((decode_kernel<BITS, 2, OUT, DEEP, SPLIT>), grid, dim3(64), 0, s, a);
    else hipLaunchKernelGGL((decode_kernel<BITS, 1, OUT, DEEP, SPLIT>), grid, dim3(64), 0, s, a);
}

// decode_kernel: a.tail_items + a.mixed_items + a.splits items per stream
// (residual, groups with partial value codes under the paper policy,
// splits), writing partials a.splits .. a.splits + a.tail_items - 1, the
// a.mixed_items after those, and 0 .. a.splits - 1.
hipError_t launch_decode(const DecodeArgs &a, hipStream_t s) {
    const int streams = a.batch * a.kv_heads;
    const int gq = a.q_heads / a.kv_heads;
    const int64_t items = (int64_t)streams * (a.splits + a.tail_items + a.mixed_items);
    if (a.items > kMaxItems || items > 0x7FFFFFFF) return hipErrorInvalidValue;
    if (a.tail_items < 1 || a.tail_chunk_step < 1 ||
        (int64_t)a.tail_items * a.tail_chunk_step < a.tail_chunks)
        return hipErrorInvalidValue;
    if (a.items != a.splits + a.tail_items + (a.mixed_groups > 0 ? a.mixed_items : 0))
        return hipErrorInvalidValue;
    if (a.n_out < 0 || a.n_out > kMaxKeyOutliers || (a.n_out > 0 && !a.outliers))
        return hipErrorInvalidValue;
    if (!side_args_ok(a.side, a.n_out)) return hipErrorInvalidValue;
    if (a.mixed_groups > 0 ? (a.mixed_items < 1 || a.mixed_step < 1 ||
                              (int64_t)a.mixed_items * a.mixed_step < a.mixed_groups)
                           : a.mixed_items != 0)
        return hipErrorInvalidValue;
    dim3 grid((unsigned)items);
    if (a.n_out > 0) {
        if (a.bits == 2) launch_decode_bits<2, true>(a, gq, grid, s);
        else if (a.bits == 8) launch_decode_bits<8, true>(a, gq, grid, s);
        else launch_decode_bits<4, true>(a, gq, grid, s);
    } else if (a.side.split) {
        if (a.bits == 2) launch_decode_bits<2, false, false, true>(a, gq, grid, s);
        else if (a.bits == 8) launch_decode_bits<8, false, false, true>(a, gq, grid, s);
        else if (a.deep) launch_decode_bits<4, false, true, true>(a, gq, grid, s);
        else launch_decode_bits<4, false, false, true>(a, gq, grid, s);
    } else if (a.bits == 2) launch_decode_bits<2>(a, gq, grid, s);
    else if (a.bits == 8) launch_decode_bits<8>(a, gq, grid, s);
    else if (a.deep) launch_decode_bits<4, false, true>(a, gq, grid, s);
    else launch_decode_bits<4>(a, gq, grid, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    launch_combine((const float *)a.part_o, (const float *)a.part_ml, a.out,
                   (int64_t)a.batch * a.q_heads, a.items, s);
    return hipGetLastError();
}

template <int BITS, bool QF32, bool OUT, bool SPLIT, int CB>
static void launch_attn_cb(const AttnArgs &a, int gq, dim3 grid, hipStream_t s) {
    const dim3 block(64 * (kAttnColBlocks / CB));
    if (gq == 4)
        hipLaunchKernelGGL((attn_kernel<BITS, 4, QF32, CB, OUT, SPLIT>), grid, block, 0, s, a);
    else if (gq == 2)
        hipLaunchKernelGGL((attn_kernel<BITS, 2, QF32, CB, OUT, SPLIT>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((attn_kernel<BITS, 1, QF32, CB, OUT, SPLIT>), grid, block, 0, s, a);
}

// Two column blocks per wavefront once the first query block is full of
// queries (T x GQ >= 128 columns): 4-5 % faster at T = 64 to 1024.  With
// fewer queries a wavefront's second block would be empty (25-33 % slower at
// T = 4 and 16), so those calls take one block per wavefront.
template <int BITS, bool QF32, bool OUT, bool SPLIT = false>
static void launch_attn_out(const AttnArgs &a, int gq, dim3 grid, hipStream_t s) {
    if (a.T * gq >= 16 * kAttnColBlocks) launch_attn_cb<BITS, QF32, OUT, SPLIT, 2>(a, gq, grid, s);
    else launch_attn_cb<BITS, QF32, OUT, SPLIT, 1>(a, gq, grid, s);
}

template <int BITS, bool QF32>
static void launch_attn_bits(const AttnArgs &a, int gq, dim3 grid, hipStream_t s) {
    if (a.n_out > 0) launch_attn_out<BITS, QF32, true>(a, gq, grid, s);
    else if (a.side.split) launch_attn_out<BITS, QF32, false, true>(a, gq, grid, s);
    else launch_attn_out<BITS, QF32, false>(a, gq, grid, s);
}

hipError_t launch_attn(const AttnArgs &a, hipStream_t s) {
    const int64_t streams = (int64_t)a.batch * a.kv_heads;
    const int gq = a.q_heads / a.kv_heads;
    const int64_t workgroups = streams * a.qblocks * a.splits;
    const int64_t rows = (int64_t)a.batch * a.q_heads * a.T;
    if (a.splits < 1 || a.splits > kMaxItems || workgroups > 0x7FFFFFFF || rows > 0x7FFFFFFF)
        return hipErrorInvalidValue;
    if (a.n_out < 0 || a.n_out > kMaxKeyOutliers || (a.n_out > 0 && !a.outliers))
        return hipErrorInvalidValue;
    if (!side_args_ok(a.side, a.n_out)) return hipErrorInvalidValue;
    const dim3 grid((unsigned)workgroups);
    if (a.bits == 2) {
        if (a.q_is_f32) launch_attn_bits<2, true>(a, gq, grid, s);
        else launch_attn_bits<2, false>(a, gq, grid, s);
    } else if (a.bits == 8) {
        if (a.q_is_f32) launch_attn_bits<8, true>(a, gq, grid, s);
        else launch_attn_bits<8, false>(a, gq, grid, s);
    } else {
        if (a.q_is_f32) launch_attn_bits<4, true>(a, gq, grid, s);
        else launch_attn_bits<4, false>(a, gq, grid, s);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.splits == 1) return e;
    launch_combine((const float *)a.part_o, (const float *)a.part_ml, a.out, rows, a.splits, s);
    return hipGetLastError();
}

}  // namespace kivi
