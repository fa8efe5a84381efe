// kivi_api.cpp -- the C ABI of libkivi (declared in include/kivi.h): config
// validation, the device-buffer layout, the n / Q(n) bookkeeping of the two
// flush policies, and stream-ordered kernel launches.
//
// Window policy ("KIVI", VeloxQuant-MLX docs, "How it works" items 3-4): the
// newest R tokens stay in full precision and aged tokens are quantized only
// in whole groups of G, so keys and values share the quantized prefix
// Q(n) = G * floor(max(0, n - R) / G).  An append from n_old to n quantizes
// tokens [Q(n_old), Q(n)) and keeps [max(Q(n), n_old), n) in the ring; the
// ring (capacity R + G) never holds more than n - Q(n) < R + G tokens.
//
// Paper policy ("[Paper review] KIVI ...", 3.2.2 and the prefill / decoding
// phases of Algorithm 1 in 3.2.3): keys keep r = n mod R tokens in full
// precision, Q_K(n) = n - r (R tokens are quantized at once when the key
// residual fills up), and values keep the newest R, Q_V(n) = max(0, n - R)
// (one token is quantized per decoding step).  Q_K >= Q_V, and the ring holds
// tokens from G * floor(Q_V / G) (the start of the value group holding Q_V,
// which is re-quantized whole as its rows arrive) to n: fewer than R + G.
#include <math.h>
#include <new>
#include <stdint.h>
#include <string.h>

#include "../../include/kivi.h"
#include "kivi_internal.h"

using namespace kivi;

static_assert(KIVI_NOALLOC_SCRATCH_BYTES == kNoAllocScratchBytes,
              "kivi.h and the kernels must agree on the fixed scratch size");

struct kivi_cache {
    kivi_config cfg;
    uint8_t *base;
    size_t bytes;
    size_t off_blocks, off_ring_k, off_ring_v, off_outliers;
    size_t off_kside;                        // split layout: key units
    int64_t max_kunits, kunit_blocks;        //   per stream; blocks per unit
    bool split;                              // G > 32: the split layout
    size_t off_seg_partial, off_seg_stats;   // segment policy scratch
    int32_t seg_chunks;                      // chunks of the longest segment
    int64_t max_groups;
    int64_t block_bytes, code_bytes;
    int64_t ring_cap;
    int esize;
    int64_t n;      // tokens cached per stream
    int64_t q;      // key tokens quantized per stream, Q(n) / Q_K(n)
    int64_t qv;     // value tokens quantized per stream (= q under the window policy)
};

namespace {

constexpr size_t kAlign = 256;
// Most decode wavefronts resident at once: 256 compute units x 16 (4 per
// SIMD, <= 128 registers per lane); decode_waves gives the plan's target.
constexpr int kMaxWaves = 4096;

// A decode pass whose blocks exceed this many bytes copies them as
// non-temporal lines: they will not stay cached until the next step anyway
// (MI355X's Infinity Cache holds 256 MiB), and streaming them saves ~8 % on
// the long-context pass.  Smaller passes keep the default policy, so that a
// step's working set can stay in the Infinity Cache for the next step.
constexpr int64_t kStreamingBytes = 128ll << 20;
// Compute units of one MI355X (the attention plan aims at two workgroups each).
constexpr int kComputeUnits = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

kivi_status validate(const kivi_config *c) {
    if (!c) return KIVI_ERR_INVALID_ARG;
    if (c->batch < 1 || c->n_kv_heads < 1 || c->n_q_heads < 1 || c->max_tokens < 1)
        return KIVI_ERR_INVALID_ARG;
    if (c->bits != 2 && c->bits != 4 && c->bits != 8) return KIVI_ERR_INVALID_ARG;
    if (c->group < 1 || c->head_dim < 1 || c->head_dim % c->group != 0) return KIVI_ERR_INVALID_ARG;
    if (c->policy == KIVI_FLUSH_SEGMENT) {
        // KCVT: values grouped over the whole head, a buffer of whole blocks
        if (c->residual <= 0 || c->residual % kGroup != 0 || c->group != c->head_dim)
            return KIVI_ERR_INVALID_ARG;
        if (c->key_outliers != 0) return KIVI_ERR_UNSUPPORTED;
    } else if (c->residual < 0 || c->residual % c->group != 0) {
        return KIVI_ERR_INVALID_ARG;
    }
    if ((int64_t)c->group * c->bits % 64 != 0) return KIVI_ERR_INVALID_ARG;
    if (c->n_q_heads % c->n_kv_heads != 0) return KIVI_ERR_INVALID_ARG;
    if (c->kv_dtype != KIVI_F16 && c->kv_dtype != KIVI_F32) return KIVI_ERR_INVALID_ARG;
    if (c->policy != KIVI_FLUSH_WINDOW && c->policy != KIVI_FLUSH_PAPER &&
        c->policy != KIVI_FLUSH_SEGMENT)
        return KIVI_ERR_INVALID_ARG;
    if (c->policy == KIVI_FLUSH_PAPER && c->residual == 0) return KIVI_ERR_INVALID_ARG;
    if (c->key_outliers < 0 || c->key_outliers > kMaxKeyOutliers) return KIVI_ERR_INVALID_ARG;
    // Shapes the kernels are built for.
    if (c->head_dim != kHeadDim) return KIVI_ERR_UNSUPPORTED;
    if (c->group != kGroup && c->group != 2 * kGroup && c->group != 4 * kGroup)
        return KIVI_ERR_UNSUPPORTED;
    const int gq = c->n_q_heads / c->n_kv_heads;
    if (gq != 1 && gq != 2 && gq != 4) return KIVI_ERR_UNSUPPORTED;
    // outlier-aware keys: built for 32-token key groups
    if (c->key_outliers > 0 && c->group != kGroup) return KIVI_ERR_UNSUPPORTED;
    if ((int64_t)c->batch * c->n_kv_heads > (1LL << 24)) return KIVI_ERR_UNSUPPORTED;
    return KIVI_OK;
}

struct Sizes {
    int64_t max_groups, block_bytes, code_bytes, ring_cap;
    int esize;
    int32_t seg_chunks;
    bool split;
    int64_t max_kunits, kunit_blocks;
    size_t off_blocks, off_kside, off_ring_k, off_ring_v, off_outliers, off_seg_partial,
        off_seg_stats, total;
};

// Block layouts.  G = 32: a block carries its key group's zero / scale and
// four value slots per token.  G > 32 (and the segment policy, whose value
// groups span all D channels), the split layout: a block carries the codes
// and its tokens' D / G value pairs only, and each key unit (a key group;
// under the segment policy one 32-token block) has its zero / scale once, in
// a region of its own, so the cache holds b bits per code and two fp16 per
// group ([NB] storage cell) and the decode reads only those bytes.
Sizes sizes_of(const kivi_config *c) {
    Sizes s;
    const int64_t streams = (int64_t)c->batch * c->n_kv_heads;
    s.max_groups = c->max_tokens / kGroup;     // 32-token blocks
    s.code_bytes = (int64_t)c->bits * kGroup * c->head_dim / 8;
    s.split = c->group > kGroup;
    s.block_bytes = s.split ? 2 * s.code_bytes + 2 * 2 * (int64_t)kGroup * (c->head_dim / c->group)
                            : 2 * s.code_bytes + 4 * (int64_t)c->head_dim * 2;
    s.kunit_blocks = c->policy == KIVI_FLUSH_SEGMENT ? 1 : c->group / kGroup;
    s.max_kunits = s.split ? (s.max_groups + s.kunit_blocks - 1) / s.kunit_blocks : 0;
    s.ring_cap = (int64_t)c->residual + c->group;
    s.esize = c->kv_dtype == KIVI_F32 ? 4 : 2;
    s.off_blocks = 0;
    s.off_kside = align_up((size_t)(streams * s.max_groups * s.block_bytes));
    s.off_ring_k = s.off_kside + align_up((size_t)(streams * s.max_kunits * 4 * c->head_dim));
    const size_t ring_bytes = align_up((size_t)(streams * s.ring_cap * c->head_dim * s.esize));
    s.off_ring_v = s.off_ring_k + ring_bytes;
    s.off_outliers = s.off_ring_v + ring_bytes;
    s.total = s.off_outliers;
    if (c->key_outliers > 0)
        s.total += align_up((size_t)(streams * s.max_groups * kOutlierRecordBytes));
    // segment policy: per-chunk statistics of the longest possible segment
    // (every block of a stream) and the per-stream statistics, float32
    s.seg_chunks = (int32_t)((s.max_groups + kSegChunkBlocks - 1) / kSegChunkBlocks);
    s.off_seg_partial = s.off_seg_stats = s.total;
    if (c->policy == KIVI_FLUSH_SEGMENT) {
        s.off_seg_partial = s.total;
        s.off_seg_stats = s.off_seg_partial + align_up((size_t)(streams * s.seg_chunks * 256 * 4));
        s.total = s.off_seg_stats + align_up((size_t)(streams * 256 * 4));
    }
    return s;
}

// Quantized prefixes of keys and values of an n-token stream.
struct Prefix {
    int64_t k, v;
};

Prefix prefix_of(const kivi_config &c, int64_t n) {
    const int64_t aged = n > c.residual ? n - c.residual : 0;
    if (c.policy == KIVI_FLUSH_PAPER) return {n - n % c.residual, aged};
    if (c.policy == KIVI_FLUSH_SEGMENT) return {n - n % c.residual, n - n % c.residual};
    const int64_t q = aged / c.group * c.group;
    return {q, q};
}

// Lowest token the ring holds: the start of the 32-token block holding Q_V
// (= Q_V under the window policy, where Q_V is a multiple of G).
int64_t ring_low(const kivi_config &, int64_t qv) { return qv / kGroup * kGroup; }

bool canonical(const kivi_cache *c) {
    const Prefix p = prefix_of(c->cfg, c->n);
    return c->q == p.k && c->qv == p.v;
}

// Where the decode and attention kernels find zero / scale.
void set_side_args(const kivi_cache *c, SideArgs &sa) {
    sa.split = c->split;
    sa.kside = c->base + c->off_kside;
    sa.max_kunits = c->max_kunits;
    int shift = 0;
    while ((1 << shift) < c->kunit_blocks) shift++;
    sa.kunit_shift = shift;
    // value slot of the 32-channel group cg: cg >> vsh of nvs slots per token
    const int gt = c->cfg.group / kGroup;
    int vsh = 0;
    while ((1 << vsh) < gt) vsh++;
    sa.vsh = c->split ? vsh : 0;
    sa.nvs = c->split ? c->cfg.head_dim / c->cfg.group : 4;
}

// G-token chunks of the residual [Q, n) (walked by one item per stream).
int64_t tail_chunks_of(const kivi_cache *c, int64_t n, int64_t q) {
    return (n - q + kGroup - 1) / kGroup;
}

struct DecodePlan {
    int32_t splits, gps;        // split items per stream, groups each
    int32_t tail_items, step;   // residual items per stream, chunks each
    bool deep;                  // three-stage split items (10 per compute unit)
};

// 4-bit passes of at least this many groups per stream run three-stage split
// items, 10 wavefronts per compute unit (2560 in one round) instead of 16 at
// two stages: measured on B32 x 131072 953 -> 868 us, while on B16 x 32768
// (1020 groups) the two-stage plan is faster (133 against 148 us).
constexpr int64_t kDeepGroups = 2048;

// Short passes (fewer groups per stream than this) aim at no more than
// kShortWaves: with ~5 groups per split a wavefront's prologue and memory
// round trips dominate, and fewer, longer splits measured faster on the
// streaming workload (8 KV x 8 batch, 262-272 groups per stream).  With the
// split prologue in 32-bit arithmetic, 3072 measured best (fused warm step
// 19.3-19.5 us; 2048: 19.6-19.7, 2560: 19.55-19.6, 3584: 19.45-19.6, 4096:
// 20.0-20.1); with the earlier 64-bit prologue 2048 had been best.
constexpr int64_t kShortGroups = 512;
constexpr int64_t kShortWaves = 3072;

// Split items aimed for per decode launch: one round of resident wavefronts.
// A wavefront's LDS (as the decode kernel declares it) is its copy stages
// (block, plus the 256-byte record with outlier-aware keys; two stages with
// records, three at 2 bits or in a deep plan, else two), at least the
// 8.5 KiB a residual item stages, plus 1 KiB of q; 160 KiB per compute unit,
// and at most 16 wavefronts (4 per SIMD, <= 128 VGPRs): 2 bits 16 per CU,
// 4 bits 14 (10 deep), 8 bits 8.  Measured against 4096 (two rounds at 8
// bits, 1.14 at 4) on B16 x 32768: 4 bits 133 -> 117 us, 8 bits 200 -> 191
// us, 8 bits with records 206 -> 198 us.  At 4 bits with records the one
// round (3328) measured slower than 4096 (148 against 140 us): 4096 is kept.
int64_t decode_waves(const kivi_config &cfg, bool deep) {
    const bool out = cfg.key_outliers > 0;
    if (out && cfg.bits == 4) return kMaxWaves;
    const int64_t block = 2 * (int64_t)cfg.bits * kGroup * cfg.head_dim / 8 + 4 * cfg.head_dim * 2;
    const int64_t stages = out ? 2 : (cfg.bits == 2 || deep) ? 3 : 2;
    int64_t lds = stages * (block + (out ? kOutlierRecordBytes : 0));
    if (lds < 8704) lds = 8704;
    lds += 1024;
    int64_t per_cu = (160 * 1024) / lds;
    if (per_cu > 16) per_cu = 16;
    return kComputeUnits * per_cu;
}

// Residual items per stream at most when each chunk is an item of its own.
constexpr int64_t kMaxTailItems = 64;

// One wavefront per work item; aim for one full round of resident
// wavefronts.  The residual of `tail_chunks` G-token chunks is one item per
// stream that walks the chunks in turn, unless the split items are so short
// (fewer than two groups per residual chunk) that the walk would outlast
// them: then each chunk is an item of its own (up to kMaxTailItems chunks),
// and the split items give up the slots.  q: tokens of the groups the split
// items cover.
DecodePlan decode_plan_of(const kivi_cache *c, int64_t q, int64_t tail_chunks) {
    const int64_t streams = (int64_t)c->cfg.batch * c->cfg.n_kv_heads;
    const int64_t ng = q / kGroup;
    const bool per_chunk_ok = tail_chunks > 1 && tail_chunks <= kMaxTailItems;
    DecodePlan p = {0, 1, 1, tail_chunks > 1 ? (int32_t)tail_chunks : 1, false};
    if (ng == 0) {
        if (per_chunk_ok) p = {0, 1, (int32_t)tail_chunks, 1, false};
        return p;
    }
    p.deep = c->cfg.bits == 4 && c->cfg.key_outliers == 0 && ng >= kDeepGroups;
    int64_t waves = decode_waves(c->cfg, p.deep);
    if (ng < kShortGroups && waves > kShortWaves) waves = kShortWaves;
    for (int pass = 0; pass < 2; pass++) {
        int64_t want = waves / streams - p.tail_items;
        if (want < 1) want = 1;
        if (want > ng) want = ng;
        const int64_t g = (ng + want - 1) / want;
        p.gps = (int32_t)g;
        p.splits = (int32_t)((ng + g - 1) / g);
        if (pass == 1 || !per_chunk_ok || g >= 2 * tail_chunks) break;
        p.tail_items = (int32_t)tail_chunks;
        p.step = 1;
    }
    return p;
}

// Residual items per stream at most (the key residual is shorter than R + G
// tokens, so it has at most (R + G) / 32 chunks of 32).
int64_t max_tail_items(const kivi_config &cfg) {
    const int64_t chunks = (cfg.residual + cfg.group) / kGroup;
    return chunks < kMaxTailItems ? chunks : kMaxTailItems;
}

// Paper policy: the groups with key codes whose value codes stop early
// (fewer than R / G + 2 of them, since Q_K - Q_V < R) are one item each, up
// to kMaxTailItems items per stream.
int64_t max_mixed_items(const kivi_config &cfg) { return max_tail_items(cfg) + 1; }

// Attention of T queries: kAttnColBlocks x 16 / GQ queries per workgroup
// (one query block), and the groups split so that about two workgroups per
// compute unit are in flight.
void attn_plan(const kivi_cache *c, int64_t T, int64_t q, int32_t *qblocks, int32_t *splits,
               int32_t *gps) {
    const int64_t streams = (int64_t)c->cfg.batch * c->cfg.n_kv_heads;
    const int gq = c->cfg.n_q_heads / c->cfg.n_kv_heads;
    const int64_t qt = 16 / gq;
    const int64_t cbs = (T + qt - 1) / qt;
    const int64_t qb = (cbs + kAttnColBlocks - 1) / kAttnColBlocks;
    *qblocks = (int32_t)qb;
    const int64_t ng = q / kGroup;
    int64_t want = 2 * kComputeUnits / (streams * qb);
    if (want < 1) want = 1;
    if (want > (ng + 3) / 4) want = (ng + 3) / 4;       // >= 4 groups per split
    if (want < 1) want = 1;
    const int64_t g = ng > 0 ? (ng + want - 1) / want : 1;
    *gps = (int32_t)g;
    *splits = ng > 0 ? (int32_t)((ng + g - 1) / g) : 1;
}

int64_t attn_max_splits(const kivi_cache *c, int64_t T) {
    const int64_t streams = (int64_t)c->cfg.batch * c->cfg.n_kv_heads;
    const int gq = c->cfg.n_q_heads / c->cfg.n_kv_heads;
    const int64_t qt = 16 / gq;
    const int64_t qb = ((T + qt - 1) / qt + kAttnColBlocks - 1) / kAttnColBlocks;
    int64_t want = 2 * kComputeUnits / (streams * qb);
    return want < 1 ? 1 : want;
}

}  // namespace

extern "C" {

const char *kivi_status_string(kivi_status s) {
    switch (s) {
    case KIVI_OK: return "ok";
    case KIVI_ERR_INVALID_ARG: return "invalid argument";
    case KIVI_ERR_UNSUPPORTED: return "unsupported shape";
    case KIVI_ERR_CAPACITY: return "capacity exceeded";
    case KIVI_ERR_BUFFER_TOO_SMALL: return "buffer too small";
    case KIVI_ERR_STATE: return "invalid state";
    case KIVI_ERR_HIP: return "HIP launch failed";
    }
    return "unknown status";
}

size_t kivi_cache_bytes(const kivi_config *cfg) {
    if (validate(cfg) != KIVI_OK) return 0;
    return sizes_of(cfg).total;
}

kivi_status kivi_cache_create(const kivi_config *cfg, void *dev_mem, size_t dev_bytes,
                              kivi_cache **out) {
    if (!out || !dev_mem) return KIVI_ERR_INVALID_ARG;
    kivi_status st = validate(cfg);
    if (st != KIVI_OK) return st;
    if ((uintptr_t)dev_mem % kAlign != 0) return KIVI_ERR_INVALID_ARG;
    const Sizes s = sizes_of(cfg);
    if (dev_bytes < s.total) return KIVI_ERR_BUFFER_TOO_SMALL;
    kivi_cache *c = new (std::nothrow) kivi_cache;
    if (!c) return KIVI_ERR_INVALID_ARG;
    c->cfg = *cfg;
    c->base = (uint8_t *)dev_mem;
    c->bytes = dev_bytes;
    c->off_blocks = s.off_blocks;
    c->off_ring_k = s.off_ring_k;
    c->off_ring_v = s.off_ring_v;
    c->off_outliers = s.off_outliers;
    c->off_kside = s.off_kside;
    c->max_kunits = s.max_kunits;
    c->kunit_blocks = s.kunit_blocks;
    c->split = s.split;
    c->off_seg_partial = s.off_seg_partial;
    c->off_seg_stats = s.off_seg_stats;
    c->seg_chunks = s.seg_chunks;
    c->max_groups = s.max_groups;
    c->block_bytes = s.block_bytes;
    c->code_bytes = s.code_bytes;
    c->ring_cap = s.ring_cap;
    c->esize = s.esize;
    c->n = 0;
    c->q = 0;
    c->qv = 0;
    *out = c;
    return KIVI_OK;
}

kivi_status kivi_cache_destroy(kivi_cache *c) {
    delete c;
    return KIVI_OK;
}

kivi_status kivi_plan_append(const kivi_cache *c, int64_t n_new, kivi_append_plan *p) {
    if (!c || !p || n_new < 0) return KIVI_ERR_INVALID_ARG;
    if (n_new > c->cfg.max_tokens - c->n) return KIVI_ERR_CAPACITY;
    const int64_t n = c->n + n_new;
    const Prefix q_new = prefix_of(c->cfg, n);
    const int64_t lo = ring_low(c->cfg, q_new.v);
    p->n_old = c->n;
    p->n_new_total = n;
    p->q_old = c->q;
    p->q_new = q_new.k;
    p->flush_token_begin = c->q;
    p->flush_token_end = q_new.k;
    p->ring_token_begin = lo > c->n ? lo : c->n;
    p->ring_token_end = n;
    p->v_flush_token_begin = c->qv;
    p->v_flush_token_end = q_new.v;
    return KIVI_OK;
}

}  // extern "C"

namespace {

// Tokens [begin, end) (all >= n_old) of every stream, copied into the ring.
RingArgs ring_args(const kivi_cache *c, const void *k, const void *v, int64_t n_new,
                   int64_t n_old, int64_t begin, int64_t end) {
    RingArgs r;
    r.in_k = k;
    r.in_v = v;
    r.n_new = n_new;
    r.n_old = n_old;
    r.ring_k = c->base + c->off_ring_k;
    r.ring_v = c->base + c->off_ring_v;
    r.ring_cap = c->ring_cap;
    r.tok_begin = begin;
    r.tok_end = end > begin ? end : begin;
    r.streams = c->cfg.batch * c->cfg.n_kv_heads;
    r.esize = c->esize;
    return r;
}

// Quantize the 32-token blocks [block_begin, block_end) of every stream:
// kinds 1 = key groups (G / 32 blocks each), 2 = value blocks, 3 = both;
// value rows at or past v_limit are left out (codes and side data 0).
// Tokens t < p.n_old are read from the ring, later ones from k / v.
// `copy` (optional): ring rows to write once every ring row the quantize
// work reads has been read, folded into its launch where one reads no ring
// row (then the copy needs no launch of its own).
kivi_status enqueue_quantize(kivi_cache *c, const kivi_append_plan &p, const void *k,
                             const void *v, int64_t n_new, int64_t block_begin,
                             int64_t block_end, int kinds, int64_t v_limit,
                             hipStream_t stream, const RingArgs *copy = nullptr) {
    if (block_end <= block_begin && !copy) return KIVI_OK;
    QuantizeArgs a;
    a.blocks = c->base + c->off_blocks;
    a.max_groups = c->max_groups;
    a.block_bytes = c->block_bytes;
    a.kside = c->base + c->off_kside;
    a.max_kunits = c->max_kunits;
    a.in_k = k;
    a.in_v = v;
    a.n_new = n_new;
    a.ring_k = c->base + c->off_ring_k;
    a.ring_v = c->base + c->off_ring_v;
    a.ring_cap = c->ring_cap;
    a.n_old = p.n_old;
    a.block_begin = block_begin;
    a.block_end = block_end;
    a.gt = c->cfg.group / kGroup;
    a.n_out = c->cfg.key_outliers;
    a.outliers = c->cfg.key_outliers > 0 ? c->base + c->off_outliers : nullptr;
    a.streams = c->cfg.batch * c->cfg.n_kv_heads;
    a.is_f32 = c->cfg.kv_dtype == KIVI_F32;
    a.bits = c->cfg.bits;
    a.kinds = kinds;
    a.v_limit = v_limit;
    a.copy = copy ? *copy : RingArgs{};
    a.quant_tasks = 0;
    a.seg_stats = nullptr;
    a.seg_partial = nullptr;
    a.seg_chunk_blocks = kSegChunkBlocks;
    a.seg_chunks = 0;
    if (kinds == 4) {
        // KCVT: the blocks [block_begin, block_end) are one segment; its key
        // statistics first, then the pairs of key and value tasks
        a.seg_stats = (float *)(c->base + c->off_seg_stats);
        a.seg_partial = (float *)(c->base + c->off_seg_partial);
        a.seg_chunks = (int32_t)((block_end - block_begin + kSegChunkBlocks - 1) / kSegChunkBlocks);
        if (block_end > block_begin && launch_segment_stats(a, stream) != hipSuccess)
            return KIVI_ERR_HIP;
    }
    return launch_quantize(a, stream) == hipSuccess ? KIVI_OK : KIVI_ERR_HIP;
}

// Everything the plan quantizes, in 32-token blocks.  Window policy: the
// tokens [q_old, q_new), keys and values together.  Paper policy: the key
// groups of [q_old, q_new), then the value blocks touched by [qv_old,
// qv_new): whole blocks, and the block holding qv_new up to that token
// (re-quantized whole on every append that adds rows to it; its earlier rows
// come out identical, since values are quantized per token).
// `copy` (optional) is written to the ring by the last of these launches.
kivi_status enqueue_flush(kivi_cache *c, const kivi_append_plan &p, const void *k, const void *v,
                          int64_t n_new, hipStream_t stream, const RingArgs *copy = nullptr) {
    const int64_t G = kGroup;
    constexpr int64_t kNoLimit = INT64_MAX;
    if (c->cfg.policy == KIVI_FLUSH_SEGMENT)
        return enqueue_quantize(c, p, k, v, n_new, p.flush_token_begin / G,
                                p.flush_token_end / G, 4, kNoLimit, stream, copy);
    if (c->cfg.policy != KIVI_FLUSH_PAPER)
        return enqueue_quantize(c, p, k, v, n_new, p.flush_token_begin / G,
                                p.flush_token_end / G, 3, kNoLimit, stream, copy);
    // paper policy: the key groups, the whole value blocks, then the value
    // block holding Q_V; the copy rides on the last of them
    const bool vflush = p.v_flush_token_end > p.v_flush_token_begin;
    const int64_t g0 = p.v_flush_token_begin / G, gw = p.v_flush_token_end / G;
    const bool vwhole = vflush && gw > g0, vpart = vflush && p.v_flush_token_end % G != 0;
    kivi_status st = enqueue_quantize(c, p, k, v, n_new, p.flush_token_begin / G,
                                      p.flush_token_end / G, 1, kNoLimit, stream,
                                      vwhole || vpart ? nullptr : copy);
    if (st != KIVI_OK) return st;
    if (vwhole) {
        st = enqueue_quantize(c, p, k, v, n_new, g0, gw, 2, kNoLimit, stream, vpart ? nullptr : copy);
        if (st != KIVI_OK) return st;
    }
    if (vpart) st = enqueue_quantize(c, p, k, v, n_new, gw, gw + 1, 2, p.v_flush_token_end, stream, copy);
    return st;
}

// Copy tokens [begin, end) (all >= n_old) of every stream into the ring.
kivi_status enqueue_ring(kivi_cache *c, const void *k, const void *v, int64_t n_new,
                         int64_t n_old, int64_t begin, int64_t end, hipStream_t stream) {
    if (end <= begin) return KIVI_OK;
    const RingArgs r = ring_args(c, k, v, n_new, n_old, begin, end);
    return launch_ring_append(r, stream) == hipSuccess ? KIVI_OK : KIVI_ERR_HIP;
}

}  // namespace

extern "C" {

// Host state (n, Q) moves only once every launch of the call was accepted.
// The launches are ordered so that a refused one leaves the old state valid:
// the ring is written only by the last launch of an append (copy
// workgroups riding on the last quantize launch, or a ring launch after all
// quantize launches), and the quantize launches before it write only
// blocks past the old prefixes (under the paper policy also the value rows
// at or past the old Q_V of the block holding it, which no call reads while
// Q_V is unchanged).
kivi_status kivi_append(kivi_cache *c, const void *k, const void *v, int64_t n_new,
                        uint32_t flags, hipStream_t stream) {
    if (!c || (flags & ~(uint32_t)KIVI_DEFER_FLUSH) != 0 || n_new < 0) return KIVI_ERR_INVALID_ARG;
    if (n_new > 0 && (!k || !v)) return KIVI_ERR_INVALID_ARG;
    kivi_append_plan p;
    kivi_status st = kivi_plan_append(c, n_new, &p);
    if (st != KIVI_OK) return st;
    if (flags & KIVI_DEFER_FLUSH) {
        // every token the next flush reads must stay addressable in the ring
        if (p.n_new_total - ring_low(c->cfg, c->qv) > c->ring_cap) return KIVI_ERR_CAPACITY;
        st = enqueue_ring(c, k, v, n_new, p.n_old, p.n_old, p.n_new_total, stream);
        if (st != KIVI_OK) return st;
        c->n = p.n_new_total;
        return KIVI_OK;
    }
    {
        // the ring copy rides on the last launch
        const RingArgs r = ring_args(c, k, v, n_new, p.n_old, p.ring_token_begin, p.ring_token_end);
        st = enqueue_flush(c, p, k, v, n_new, stream, &r);
    }
    if (st != KIVI_OK) return st;
    c->n = p.n_new_total;
    c->q = p.q_new;
    c->qv = p.v_flush_token_end;
    return KIVI_OK;
}

kivi_status kivi_flush(kivi_cache *c, hipStream_t stream) {
    if (!c) return KIVI_ERR_INVALID_ARG;
    kivi_append_plan p;
    kivi_status st = kivi_plan_append(c, 0, &p);
    if (st != KIVI_OK) return st;
    // n_old == n: every token to quantize is read from the ring
    st = enqueue_flush(c, p, c->base + c->off_ring_k, c->base + c->off_ring_v, 0, stream);
    if (st != KIVI_OK) return st;
    c->q = p.q_new;
    c->qv = p.v_flush_token_end;
    return KIVI_OK;
}

size_t kivi_decode_workspace_bytes(const kivi_cache *c) {
    if (!c) return 0;
    // decode_plan_of never makes more than max(1, kMaxWaves / streams - 1)
    // split items per stream, whatever n is (fewer when the residual takes
    // one item per chunk), plus at most one residual item per chunk, and
    // under the paper policy one item for the groups with partial value codes.
    const int64_t streams = (int64_t)c->cfg.batch * c->cfg.n_kv_heads;
    int64_t splits = kMaxWaves / streams - 1;
    if (splits < 1) splits = 1;
    const int64_t items = splits + max_tail_items(c->cfg) +
                          (c->cfg.policy == KIVI_FLUSH_PAPER ? max_mixed_items(c->cfg) : 0);
    const int64_t bhq = (int64_t)c->cfg.batch * c->cfg.n_q_heads;
    return (size_t)(bhq * items * (c->cfg.head_dim + 2) * 4);
}

kivi_status kivi_decode_plan(const kivi_cache *c, int32_t *splits, int32_t *gps) {
    if (!c || !splits || !gps) return KIVI_ERR_INVALID_ARG;
    const DecodePlan p = decode_plan_of(c, ring_low(c->cfg, c->qv), tail_chunks_of(c, c->n, c->q));
    *splits = p.splits;
    *gps = p.gps;
    return KIVI_OK;
}

}  // extern "C"

namespace {

kivi_status check_decode_args(const kivi_cache *c, const void *q, int32_t q_dtype,
                              const float *out, const void *workspace, size_t ws_bytes) {
    if (!c || !q || !out || !workspace) return KIVI_ERR_INVALID_ARG;
    if (q_dtype != KIVI_F16 && q_dtype != KIVI_F32) return KIVI_ERR_INVALID_ARG;
    if (ws_bytes < kivi_decode_workspace_bytes(c)) return KIVI_ERR_BUFFER_TOO_SMALL;
    return KIVI_OK;
}

// The decode launches over the cache's current (canonical) state.  Tokens
// t >= in_from (in_from = n - in_n) were appended by the same call and are
// still only in in_k / in_v: the residual items read them there and copy
// them into the ring.
kivi_status enqueue_decode(kivi_cache *c, const void *q, int32_t q_dtype, float softmax_scale,
                           float *out, void *workspace, hipStream_t stream, const void *in_k,
                           const void *in_v, int64_t in_n, int64_t in_from) {
    DecodeArgs a;
    // groups [0, nq / G): key and value codes (split items); [nq, q): key
    // codes, value codes below qv (paper policy only); [q, n): the residual
    const int64_t nq = ring_low(c->cfg, c->qv);
    const int32_t mixed = (int32_t)((c->q - nq) / kGroup);
    const int64_t chunks = tail_chunks_of(c, c->n, c->q);
    const DecodePlan plan = decode_plan_of(c, nq, chunks);
    const int64_t bhq = (int64_t)c->cfg.batch * c->cfg.n_q_heads;
    const int32_t mixed_items = mixed <= kMaxTailItems ? mixed : (int32_t)kMaxTailItems;
    const int32_t mixed_step = mixed > 0 ? (mixed + mixed_items - 1) / mixed_items : 1;
    const int64_t items = plan.splits + plan.tail_items + (mixed > 0 ? mixed_items : 0);
    a.blocks = c->base + c->off_blocks;
    a.max_groups = c->max_groups;
    a.block_bytes = c->block_bytes;
    set_side_args(c, a.side);
    a.ring_k = c->base + c->off_ring_k;
    a.ring_v = c->base + c->off_ring_v;
    a.ring_cap = c->ring_cap;
    a.ring_is_f32 = c->cfg.kv_dtype == KIVI_F32;
    a.q = q;
    a.q_is_f32 = q_dtype == KIVI_F32;
    a.out = out;
    a.part_o = (float *)workspace;
    a.part_ml = (float *)workspace + bhq * items * c->cfg.head_dim;
    a.batch = c->cfg.batch;
    a.kv_heads = c->cfg.n_kv_heads;
    a.q_heads = c->cfg.n_q_heads;
    a.bits = c->cfg.bits;
    a.n_tokens = c->n;
    a.n_quant = nq;
    a.n_tail = c->q;
    a.n_vquant = c->qv;
    a.mixed_groups = mixed;
    a.mixed_items = mixed > 0 ? mixed_items : 0;
    a.mixed_step = mixed_step;
    a.splits = plan.splits;
    a.groups_per_split = plan.gps;
    a.deep = plan.deep;
    a.tail_chunks = (int32_t)chunks;
    a.tail_items = plan.tail_items;
    a.tail_chunk_step = plan.step;
    a.items = (int32_t)items;
    const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)c->cfg.head_dim);
    a.sm_log2 = scale * 1.4426950408889634f;
    a.n_out = c->cfg.key_outliers;
    a.outliers = c->cfg.key_outliers > 0 ? c->base + c->off_outliers : nullptr;
    a.in_k = in_k;
    a.in_v = in_v;
    a.in_n = in_n;
    a.in_from = in_from;
    {
        const int64_t rec = c->cfg.key_outliers > 0 ? kOutlierRecordBytes : 0;
        const int64_t pass = (int64_t)c->cfg.batch * c->cfg.n_kv_heads * (nq / kGroup) *
                             (c->block_bytes + rec);
        a.nt = pass > kStreamingBytes;
    }
    if (launch_decode(a, stream) != hipSuccess) return KIVI_ERR_HIP;
    return KIVI_OK;
}

}  // namespace

extern "C" {

kivi_status kivi_decode_attn(kivi_cache *c, const void *q, int32_t q_dtype, float softmax_scale,
                             float *out, void *workspace, size_t ws_bytes, hipStream_t stream) {
    kivi_status st = check_decode_args(c, q, q_dtype, out, workspace, ws_bytes);
    if (st != KIVI_OK) return st;
    if (c->n == 0 || !canonical(c)) return KIVI_ERR_STATE;
    return enqueue_decode(c, q, q_dtype, softmax_scale, out, workspace, stream, nullptr, nullptr,
                          0, INT64_MAX);
}

kivi_status kivi_append_decode(kivi_cache *c, const void *k, const void *v, int64_t n_new,
                               const void *q, int32_t q_dtype, float softmax_scale, float *out,
                               void *workspace, size_t ws_bytes, hipStream_t stream) {
    if (!c || n_new < 0 || (n_new > 0 && (!k || !v))) return KIVI_ERR_INVALID_ARG;
    kivi_status st = check_decode_args(c, q, q_dtype, out, workspace, ws_bytes);
    if (st != KIVI_OK) return st;
    if (!canonical(c)) return KIVI_ERR_STATE;
    kivi_append_plan p;
    st = kivi_plan_append(c, n_new, &p);
    if (st != KIVI_OK) return st;
    if (p.n_new_total == 0) return KIVI_ERR_STATE;
    const bool quantizes = p.flush_token_end > p.flush_token_begin ||
                           p.v_flush_token_end > p.v_flush_token_begin;
    if (n_new == 0 || quantizes || c->cfg.policy != KIVI_FLUSH_WINDOW) {
        // the append's own launches, then the decode over the ring
        st = kivi_append(c, k, v, n_new, 0, stream);
        if (st != KIVI_OK) return st;
        return enqueue_decode(c, q, q_dtype, softmax_scale, out, workspace, stream, nullptr,
                              nullptr, 0, INT64_MAX);
    }
    // nothing ages out: every new row lands in the residual, and the decode's
    // residual items take it from k / v and write it into the ring.  The
    // decode plan is made for the new n; if its launch is refused nothing was
    // enqueued, and n goes back to its old value.
    c->n = p.n_new_total;
    st = enqueue_decode(c, q, q_dtype, softmax_scale, out, workspace, stream, k, v, n_new,
                        p.n_old);
    if (st != KIVI_OK) c->n = p.n_old;
    return st;
}

kivi_status kivi_decode_attn_noalloc(kivi_cache *c, const void *q, int32_t q_dtype,
                                     float softmax_scale, float *out, hipStream_t stream) {
    if (!c || !q || !out) return KIVI_ERR_INVALID_ARG;
    if (q_dtype != KIVI_F16 && q_dtype != KIVI_F32) return KIVI_ERR_INVALID_ARG;
    if (kivi_decode_workspace_bytes(c) > KIVI_NOALLOC_SCRATCH_BYTES) return KIVI_ERR_BUFFER_TOO_SMALL;
    if (c->n == 0 || !canonical(c)) return KIVI_ERR_STATE;
    void *ws = nullptr;
    if (noalloc_scratch(&ws) != hipSuccess) return KIVI_ERR_HIP;
    return enqueue_decode(c, q, q_dtype, softmax_scale, out, ws, stream, nullptr, nullptr, 0,
                          INT64_MAX);
}

size_t kivi_attn_workspace_bytes(const kivi_cache *c, int64_t T) {
    if (!c || T < 1) return 0;
    const int64_t splits = attn_max_splits(c, T);
    if (splits <= 1) return 0;
    const int64_t rows = (int64_t)c->cfg.batch * c->cfg.n_q_heads * T;
    return (size_t)(rows * splits * (c->cfg.head_dim + 2) * 4);
}

kivi_status kivi_attn(kivi_cache *c, const void *q, int32_t q_dtype, int64_t T, int32_t causal,
                      float softmax_scale, float *out, void *workspace, size_t ws_bytes,
                      hipStream_t stream) {
    if (!c || !q || !out || T < 1) return KIVI_ERR_INVALID_ARG;
    if (q_dtype != KIVI_F16 && q_dtype != KIVI_F32) return KIVI_ERR_INVALID_ARG;
    if (causal != 0 && causal != 1) return KIVI_ERR_INVALID_ARG;
    if (c->n == 0 || !canonical(c)) return KIVI_ERR_STATE;
    if (causal && T > c->n) return KIVI_ERR_INVALID_ARG;
    const int64_t q_full = ring_low(c->cfg, c->qv);     // groups with value codes
    const int64_t rows = (int64_t)c->cfg.batch * c->cfg.n_q_heads * T;
    if (rows > 0x7FFFFFFF) return KIVI_ERR_UNSUPPORTED;
    const size_t need = kivi_attn_workspace_bytes(c, T);
    if (need > 0 && (!workspace || ws_bytes < need)) return KIVI_ERR_BUFFER_TOO_SMALL;
    AttnArgs a;
    int32_t qblocks, splits, gps;
    attn_plan(c, T, q_full, &qblocks, &splits, &gps);
    a.blocks = c->base + c->off_blocks;
    a.max_groups = c->max_groups;
    a.block_bytes = c->block_bytes;
    set_side_args(c, a.side);
    a.ring_k = c->base + c->off_ring_k;
    a.ring_v = c->base + c->off_ring_v;
    a.ring_cap = c->ring_cap;
    a.ring_f32 = c->cfg.kv_dtype == KIVI_F32;
    a.q = q;
    a.q_is_f32 = q_dtype == KIVI_F32;
    a.out = out;
    a.part_o = (float *)workspace;
    a.part_ml = splits > 1 ? (float *)workspace + rows * splits * c->cfg.head_dim : nullptr;
    a.batch = c->cfg.batch;
    a.kv_heads = c->cfg.n_kv_heads;
    a.q_heads = c->cfg.n_q_heads;
    a.bits = c->cfg.bits;
    a.n_tokens = c->n;
    a.n_quant = c->q;
    a.n_vquant = c->qv;
    a.T = T;
    a.causal = causal;
    a.qblocks = qblocks;
    a.splits = splits;
    a.groups_per_split = gps;
    const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)c->cfg.head_dim);
    a.sm_log2 = scale * 1.4426950408889634f;
    a.n_out = c->cfg.key_outliers;
    a.outliers = c->cfg.key_outliers > 0 ? c->base + c->off_outliers : nullptr;
    if (launch_attn(a, stream) != hipSuccess) return KIVI_ERR_HIP;
    return KIVI_OK;
}

kivi_status kivi_attn_plan(const kivi_cache *c, int64_t T, int32_t *qblocks, int32_t *splits,
                           int32_t *groups_per_split) {
    if (!c || T < 1 || !qblocks || !splits || !groups_per_split) return KIVI_ERR_INVALID_ARG;
    attn_plan(c, T, ring_low(c->cfg, c->qv), qblocks, splits, groups_per_split);
    return KIVI_OK;
}

kivi_status kivi_get_layout(const kivi_cache *c, kivi_layout *o) {
    if (!c || !o) return KIVI_ERR_INVALID_ARG;
    o->blocks = c->off_blocks;
    o->ring_k = c->off_ring_k;
    o->ring_v = c->off_ring_v;
    o->block_bytes = (size_t)c->block_bytes;
    o->code_bytes = (size_t)c->code_bytes;
    o->off_kcode = 0;
    o->off_vcode = (size_t)c->code_bytes;
    if (c->split) {
        // key zero / scale inside a key unit; value pairs after the codes
        o->off_kscale = 0;
        o->off_kzero = 2 * (size_t)c->cfg.head_dim;
        o->off_vscale = 2 * (size_t)c->code_bytes;
        o->off_vzero = o->off_vscale + 2 * (size_t)kGroup * (c->cfg.head_dim / c->cfg.group);
    } else {
        o->off_kscale = 2 * (size_t)c->code_bytes;
        o->off_kzero = o->off_kscale + 2 * (size_t)c->cfg.head_dim;
        o->off_vscale = o->off_kzero + 2 * (size_t)c->cfg.head_dim;
        o->off_vzero = o->off_vscale + 2 * (size_t)c->cfg.head_dim;
    }
    o->kside = c->split ? c->off_kside : 0;
    o->kside_unit_tokens = c->split ? c->kunit_blocks * kGroup : 0;
    o->max_kside_units = c->max_kunits;
    o->max_groups = c->max_groups;
    o->ring_capacity = c->ring_cap;
    o->n_tokens = c->n;
    o->n_quantized = c->q;
    o->n_vquantized = c->qv;
    o->outliers = c->cfg.key_outliers > 0 ? c->off_outliers : 0;
    return KIVI_OK;
}

}  // extern "C"
