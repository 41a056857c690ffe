// Internal interface between the C-ABI host code and the HIP kernels.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace pda {

// What a fold launch writes.
enum FoldMode : int {
    kModePartial = 0,  // split-K partial (o, m, l) into the workspace
    kModeFinal = 1,    // single split: BF16 o / l straight to the output
    kModeTiled = 2,    // fold a tile into the persistent (m, l, o) state
};

// Arguments of one fold launch (passed by value as the kernel argument).
struct FoldParams {
    const uint16_t* q;       // bf16 [S, nq, D]
    const uint16_t* k;       // K pool: bf16, or E4M3 bytes (FP8 cache)
    const uint16_t* v;       // V pool, same element type
    const int32_t* tables;   // block tables [S, table_stride] (one-shot) or
                             // tile blocks [S, tile_capacity] (tiled)
    const int32_t* lens;     // seq_lens [S] (one-shot) or tile block counts [S]
    float* ws;               // workspace (partial) or m state (tiled)
    float* l_state;          // tiled only
    float* o_state;          // tiled only
    uint16_t* out;           // final only: bf16 [S, nq, D]
    int64_t blk_s, tok_s, kvh_s;   // element strides of the pools
    uint32_t num_blocks;     // blocks in the pools; ids outside are dropped
    int nq, nkv, G, HG;      // heads, GQA ratio, head groups per KV head
    int bs, table_stride;
    int nsplit;              // splits per sequence (one-shot)
    int lbvs;                // valid slots of a tile's last block (tiled)
    float c;                 // scale * log2(e) (times k_scale for an FP8 cache)
    float v_scale;           // FP8 cache only: V = decode(v8) * v_scale
    // Parts: `parts` workgroups share one item (one split of one sequence
    // and head group, or one sequence's tile), of which an item of n blocks
    // uses min(parts, ceil(n / part_min)), each folding a contiguous run of
    // its blocks into a record of `sub`; the last to arrive (ticket in
    // `tick`) combines the records in part order and writes what one
    // workgroup would.  parts == 1: no records, no tickets.  Null sub /
    // tick: the library's own device arrays (kPartSubFloats / kPartTickets
    // entries).
    int parts;
    int part_min;            // blocks per part at least (parts > 1)
    float* sub;              // [item][part] records (part_rec_floats each)
    uint32_t* tick;          // [item] arrival counters, 0 between launches
};

// Ordering of the part hand-over (record stores, ticket, record loads).
// 0 (default): every record store is an agent-scope atomic store (it writes
// through the XCD's non-coherent L2), each thread waits for its stores to
// be acknowledged (s_waitcnt 0) before the workgroup barrier, one thread
// then takes the ticket with a relaxed agent-scope atomic (performed at the
// device-coherent level), and the combining workgroup reads the records
// with agent-scope atomic loads issued only after the ticket value has
// come back through LDS and a barrier (the barrier's workgroup fences keep
// the compiler from moving the loads above it).  Correctness rests on that
// hardware ordering, not on a release / acquire pair of the memory model.
// 1: the ticket is an agent-scope acquire-release RMW and the combiner
// fences (acquire); 2: the combiner alone fences (acquire).  Both are
// formally ordered and measured slower on MI355X (L2 writeback /
// invalidate per workgroup): the 131072-token sequence +14 % / +12 %, the
// packed batch +12 % / +2.4 %, the tiled step +32 % / +5 %.
#ifndef PDA_PARTS_ORDER
#define PDA_PARTS_ORDER 0
#endif
// Heads one fold workgroup carries at most (the packed width).
constexpr int kMaxHeadsPerGroup = 8;

// Most parts per item, and the capacity of the library's own part arrays.
// A one-shot item uses no more parts than it has runs of kMinPartBlocks
// blocks (the packed kernel likewise); a tile, runs of kMinTilePartBlocks.
constexpr int kMaxParts = 8;
constexpr int kMinPartBlocks = 32;
constexpr int kMinTilePartBlocks = 16;
constexpr uint64_t kPartTickets = 1u << 16;
constexpr uint64_t kPartSubFloats = 1u << 22;   // 16 MiB
// Floats of one part record for gc heads of head_dim d: o [gc][d], m [gc],
// l [gc], padded to whole 128-byte lines so that no two records share one.
constexpr uint64_t part_rec_floats(int gc, int d) {
    return ((uint64_t)gc * (d + 2) + 31) / 32 * 32;
}

// LDS bytes a fold workgroup of `waves` waves needs.
size_t fold_lds_bytes(int head_dim, int gc, int waves);

// Most waves a fold workgroup for gc heads may have (its launch bound).
int fold_max_waves(int gc);

// Launches the fold kernel for (mode, head_dim, gc) on grid x = `grid_x`,
// y = number of sequences.  head_dim in {64, 128, 256}, gc in 1..8.
hipError_t launch_fold(int mode, int head_dim, int gc, const FoldParams& p, uint32_t grid_x,
                       uint32_t grid_y, int waves, hipStream_t stream, bool kv8 = false);

// Split-K merge: workspace -> bf16 out.
hipError_t launch_merge(const float* ws, uint16_t* out, uint32_t num_seqs, int nq, int head_dim,
                        int nsplit, hipStream_t stream);

// Tiled state fill (m, l, o := -inf, 0, 0) and finalize.
hipError_t launch_tiled_begin(float* m, float* l, float* o, uint64_t n_q, int head_dim,
                              hipStream_t stream);
hipError_t launch_tiled_finalize(const float* l, const float* o, uint16_t* out, uint64_t n_q,
                                 int head_dim, hipStream_t stream);

// GQA-packed MFMA decode (8 q heads x head_dim 256 per workgroup): one
// split writes bf16 out; nsplit > 1 writes split-K partials to ws.
struct PackedParams {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const int32_t* tables;
    const int32_t* lens;
    uint16_t* out;           // nsplit == 1
    float* ws;               // nsplit > 1
    int64_t blk_s, tok_s, kvh_s;
    uint32_t num_blocks;
    int nq, nkv;
    int bs, table_stride;
    int nsplit;
    float c;                 // scale * log2(e) (times k_scale for an FP8 cache)
    float v_scale;           // FP8 cache: V = decode(v) * v_scale
    int parts;               // nsplit == 1: workgroups per (sequence, KV head);
                             // 1, or up to kMaxParts with the library's records
};
// Sequences one packed launch with `parts` parts may carry (the library's
// part records and tickets).
uint32_t packed_part_rows(uint32_t nkv, int parts);
// kv8: k and v hold OCP E4M3 bytes (strides in bytes).
hipError_t launch_packed(const PackedParams& p, uint32_t num_seqs, hipStream_t stream,
                         bool kv8 = false);

// Causal paged prefill of one sequence, head_dim 256 (MFMA).
struct PrefillParams {
    const uint16_t* q;       // bf16 [q_len, nq, 256]
    const uint16_t* k;       // bf16 K pool
    const uint16_t* v;       // bf16 V pool
    const int32_t* table;    // block table of the sequence
    uint16_t* out;           // bf16 [q_len, nq, 256]
    int64_t blk_s, tok_s;    // element strides of the pools
    uint32_t num_blocks;
    int nq, nkv, bs;
    int q_len, kv_len, q_offset;
    float c;                 // scale * log2(e)
};
hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream);

}  // namespace pda
