// Private interface between the C-ABI front end (kivi_api.cpp) and the HIP
// kernels (kivi_kernels.hip).  Not installed, not part of the ABI.
#pragma once
#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

namespace kivi {

constexpr int kHeadDim = 128;   // D: channels per head
constexpr int kGroup = 32;      // tokens per block (G: 32, 64 or 128 per key / value group)
constexpr int kMaxKeyOutliers = 3;        // fp16 key channels per key group at most
constexpr int kOutlierRecordBytes = 256;  // per block: uint16 channel[3], pad, fp16 [3][32]

// Copy tokens [tok_begin, tok_end) of every stream from the appended chunk
// into the ring.
struct RingArgs {
    const void *in_k, *in_v;
    int64_t n_new, n_old;
    void *ring_k, *ring_v;
    int64_t ring_cap;
    int64_t tok_begin, tok_end;
    int32_t streams;
    int32_t esize;              // bytes per element (2 or 4)
};

// Quantize the 32-token blocks [block_begin, block_end) of every stream.  A
// key group spans gt = G / 32 blocks (block_begin and block_end are then
// multiples of gt for key tasks); a value group spans 32 * gt channels of one
// token.  Token t < n_old is read from ring slot t % ring_cap, later tokens
// from row (t - n_old) of the appended chunk.
struct QuantizeArgs {
    uint8_t *blocks;            // [streams][max_groups][block_bytes]
    int64_t max_groups;
    int64_t block_bytes;
    // Split layout (G > 32): key units [streams][max_kunits][2][D] fp16, one
    // per key group (segment policy: per block); blocks carry the codes and
    // D / G value pairs per token.
    uint8_t *kside;
    int64_t max_kunits;
    const void *in_k, *in_v;    // [streams][n_new][D] chunk (kv dtype)
    int64_t n_new;
    const void *ring_k, *ring_v;// [streams][ring_cap][D] (kv dtype)
    int64_t ring_cap;
    int64_t n_old;
    int64_t block_begin, block_end;
    int32_t streams;
    int32_t is_f32;             // kv dtype: 0 fp16, 1 fp32
    int32_t bits;               // 2, 4 or 8
    int32_t gt;                 // blocks per key group: G / 32 (1, 2 or 4)
    int32_t n_out;              // fp16 key channels per key group (0: none)
    uint8_t *outliers;          // [streams][max_groups][kOutlierRecordBytes]
    int32_t kinds;              // 1: key groups, 2: value blocks, 3: both, 4: segment
                                // pairs (per block a key task with the segment's
                                // statistics, then a value task)
    int64_t v_limit;            // value codes / side data of tokens >= v_limit are written 0
    // Rows to copy into the ring as well (none when copy.tok_end <= tok_begin).
    // The launch that reads no ring row does the copy in extra workgroups,
    // after its quant_tasks workgroups; without one, a ring append follows.
    RingArgs copy;
    uint32_t quant_tasks;       // set by the launcher
    // Segment policy (KCVT): the key statistics of the blocks [block_begin,
    // block_end) taken as one segment: seg_stats [streams][256] = per-channel
    // minimum [128] and maximum [128] (float32), computed by
    // launch_segment_stats through seg_partial [streams][seg_chunks][256]
    // (seg_chunk_blocks blocks per chunk).
    float *seg_stats;
    float *seg_partial;
    int32_t seg_chunk_blocks;
    int32_t seg_chunks;
};

// Blocks per wavefront of the segment statistics pass.
constexpr int kSegChunkBlocks = 16;

// Where the decode and attention kernels find zero / scale.  G = 32: in
// every block (kscale, kzero, then four value slots per token).  Split
// layout (split = 1): key units of 2 x D fp16 in kside (unit = block >>
// kunit_shift), nvs value slots per token after the block's codes.  The
// 32-channel group cg reads value slot cg >> vsh of nvs.
struct SideArgs {
    int32_t split;
    const uint8_t *kside;       // [streams][max_kunits][2][D] fp16
    int64_t max_kunits;
    int32_t kunit_shift;
    int32_t vsh, nvs;
};

struct DecodeArgs {
    const uint8_t *blocks;
    int64_t max_groups;
    int64_t block_bytes;
    SideArgs side;
    const void *ring_k, *ring_v;
    int64_t ring_cap;
    int32_t ring_is_f32;
    const void *q;              // [B][Hq][D]
    int32_t q_is_f32;
    float *out;                 // [B][Hq][D] float32
    float *part_o;              // [B*Hq][n_items_per_stream][D]
    float *part_ml;             // [B*Hq][n_items_per_stream][2]  (m log2, l)
    int32_t batch, kv_heads, q_heads;
    int32_t bits;
    int32_t n_out;              // fp16 key channels per group (0: none)
    const uint8_t *outliers;    // [streams][max_groups][kOutlierRecordBytes]
    int64_t n_tokens;           // n
    int64_t n_quant;            // groups [0, n_quant / G) hold key and value codes
    int64_t n_tail;             // fp16 keys and values from here to n (the residual)
    int64_t n_vquant;           // value codes exist for tokens < n_vquant
    int32_t mixed_groups;       // groups from n_quant / G on with key codes but value
                                // codes only below n_vquant (paper policy; else 0)
    int32_t mixed_items;        // items per stream over them (each takes mixed_step
    int32_t mixed_step;         //   consecutive groups)
    int32_t splits;             // work items per stream over quantized groups
    int32_t groups_per_split;
    int32_t tail_chunks;        // G-token chunks of the residual
    int32_t tail_items;         // residual items per stream (each walks tail_chunk_step
    int32_t tail_chunk_step;    //   consecutive chunks)
    int32_t items;              // partials per (batch, query head): splits, residual, mixed
    float sm_log2;              // softmax scale * log2(e)
    // Rows appended by the same call (append + decode in one launch): tokens
    // t >= in_from are read from in_k / in_v ([streams][in_n][D], kv dtype)
    // instead of the ring, and the residual items also write them into the
    // ring.  in_from = INT64_MAX when every residual row is in the ring.
    const void *in_k, *in_v;
    int64_t in_n, in_from;
    int32_t nt;                 // split items copy their blocks as non-temporal lines
    int32_t deep;               // 4 bits, no outliers: three-stage split items
};

// Attention of T queries per (batch, query head) over the cache.  One
// workgroup per (stream, query block, split): its wavefronts each take 16/GQ
// queries x GQ heads and share the K/V blocks of the split's groups; the
// last split also walks the fp16 residual.
struct AttnArgs {
    const uint8_t *blocks;
    int64_t max_groups;
    int64_t block_bytes;
    SideArgs side;
    const void *ring_k, *ring_v;  // ring rows, fp16 or (ring_f32) float32
    int64_t ring_cap;
    int32_t ring_f32;
    const void *q;              // [B][Hq][T][D]
    int32_t q_is_f32;
    float *out;                 // [B][Hq][T][D] float32
    float *part_o;              // [B*Hq*T][splits][D] (splits > 1)
    float *part_ml;             // [B*Hq*T][splits][2]  (m log2, l)
    int32_t batch, kv_heads, q_heads;
    int32_t bits;
    int64_t n_tokens, n_quant;  // n, Q(n) (Q_K under the paper policy)
    int64_t n_vquant;           // value tokens quantized (Q_V; = n_quant, window policy)
    int64_t T;                  // queries per (batch, query head)
    int32_t causal;             // query t is token n - T + t and sees tokens <= it
    int32_t qblocks;            // query blocks per stream
    int32_t splits;             // group ranges per (stream, query block)
    int32_t groups_per_split;
    float sm_log2;              // softmax scale * log2(e)
    int32_t n_out;              // outlier-aware keys: channels per key group kept in fp16
    const uint8_t *outliers;    // [streams][max_groups][kOutlierRecordBytes] (n_out > 0)
};

// Bytes of the fixed device array that holds the decode partials of
// kivi_decode_attn_noalloc (KIVI_NOALLOC_SCRATCH_BYTES in kivi.h).
constexpr size_t kNoAllocScratchBytes = (size_t)32 << 20;

// Device address of that array on the current device (looked up with
// hipGetSymbolAddress on the first call per device, then cached).
hipError_t noalloc_scratch(void **ptr);

hipError_t launch_quantize(const QuantizeArgs &a, hipStream_t s);
// Per-channel key minimum and maximum over the blocks [block_begin,
// block_end) of every stream into a.seg_stats (two launches: chunks, then a
// reduction per stream).
hipError_t launch_segment_stats(const QuantizeArgs &a, hipStream_t s);
hipError_t launch_ring_append(const RingArgs &a, hipStream_t s);
hipError_t launch_decode(const DecodeArgs &a, hipStream_t s);
hipError_t launch_attn(const AttnArgs &a, hipStream_t s);

// Attention of T queries: a workgroup covers kAttnColBlocks 16-column blocks
// (one query block, 128 columns) and reads each cache block once.  Its
// wavefronts take CB column blocks each (kAttnColBlocks / CB wavefronts):
// CB = 2 unpacks a block's codes once for two column blocks (~220 VGPRs, 2
// wavefronts per SIMD); CB = 1 (8 wavefronts) serves calls whose first query
// block is not full, where a second column block would be empty work.
constexpr int kAttnColBlocks = 8;

}  // namespace kivi
