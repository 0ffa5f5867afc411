// internal.h -- launch plan shared by the host API (api.cpp) and the HIP
// kernels.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace slimkv {

constexpr int kHeadDim = 128;
constexpr int kWaves = 4;              // waves per attention workgroup
constexpr int kThreads = 64 * kWaves;  // attention workgroup size
constexpr int kMaxGroup = 8;           // query heads per KV head (G)
constexpr int kMaxChunks = 64;         // workgroups per unit (each writes one partial slot)
constexpr int kCounterStride = 16;     // uint32 per unit's counters: one 64-byte line each
constexpr int kWgPerCu = 2;            // resident attention workgroups per CU the grid targets
#ifndef SLIMKV_ATTN_DEPTH
#define SLIMKV_ATTN_DEPTH 1
#endif
constexpr int kAttnDepth = SLIMKV_ATTN_DEPTH;  // tile depth of the uniform bf16 attention kernel
constexpr int kMaxRaggedBatch = 1024;  // sequences per ragged call (their lengths sit in LDS)
constexpr int kMaxPageEntries = 4096;  // page-table entries of one sequence (staged in LDS)
constexpr int kMinPageShift = 6;       // pages hold at least 64 rows: no tile spans two pages
constexpr int kMaxPageShift = 16;
constexpr int kChunkRows = 16;         // query rows (tokens x heads) per unit in chunk calls
constexpr int kChunkMaxSlots = 2048;   // workgroup slots a chunk call is shaped for, at most
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;  // device scratch of the no-alloc entry point
constexpr size_t kWsHeader = 256;      // workspace bytes before the counters: word 0 is the
                                       // status SLIMKV_FLAG_CHECK_WORKSPACE reports in

enum SegKind : int32_t {
  kSegLatent = 0,  // beacon rows: keys of width r_K scored with the latent
                   // query, values of width r_V summed in latent space
  kSegFull = 1,    // full-width rows (raw window, rebuilt beacons, full KV)
};

// One run of rows that every (b, kv head) unit owns, e.g. its N_b beacons.
struct Segment {
  const void* K;       // [B, H_kv, rows, rk]
  const void* V;       // [B, H_kv, rows, rv]
  int32_t kind;        // SegKind
  int32_t rows;        // rows per unit (0: the segment is absent)
  int32_t rk, rv;      // row widths in elements (d for kSegFull)
  int32_t row_bytes;   // (rk + rv) * element bytes
  int32_t tile;        // tile height (rows) the segment is swept in
};

// Everything the attention kernel reads.  seg[0] holds each unit's beacon
// rows, seg[1] its full-width raw rows.  `chunks` workgroups share a unit's
// rows tile by tile; each writes one partial slot (empty ones included) and
// the last workgroup of a unit merges all of them.
struct AttnArgs {
  Segment seg[2];
  int32_t batch, num_q_heads, num_kv_heads, group;
  int32_t chunks;         // workgroups per unit (grid = units * chunks)
  int32_t deterministic;  // 1: tiles dealt round-robin (default), 0: from the counter
  int64_t unit_bytes;     // cache bytes per unit over both segments
  int32_t rank_v;         // r_V of a latent beacon segment (0 if none)
  const void* q;          // [B, H_q, d] before rotation
  const int32_t* q_pos;   // [B]
  const void* U_K;        // [H_kv, d, r_K] (latent segment only)
  const void* U_V;        // [H_kv, d, r_V] (latent segment only)
  double score_scale;     // scale * log2(e): scores are kept in log2 units
  double inv_freq_pow2[6];  // theta^(-2 * 2^k / d), k = 0..5, on the host in fp64:
                            // theta^(-2i/d) is the product over i's set bits
  int32_t rank_k;         // r_K of a latent beacon segment (0 if none)
  uint32_t* counters;     // [units][kCounterStride]: workgroups done, tiles handed out
                          // (zero between calls)
  uint32_t* flags;        // [partial slots]: 1 while a slot holds a published partial the
                          // unit's merge has not read (zero between calls)
  float* part_ml;         // [units, chunks, G, 2]  (max, sum of exp), log2 units
  float* part_acc;        // [units, chunks, G, d]  exp-weighted value sums
  float* out;             // [B, H_q, d]
  float* lse;             // [B, H_q] or null
  // Ragged calls only (seg[0].rows, seg[1].rows are then the capacities,
  // i.e. the row strides of each unit's arrays):
  const int32_t* seq_beacons;  // [B] live beacon rows per sequence, or null (all)
  const int32_t* seq_raw;      // [B] live raw rows before the new token, or null (all)
  const void* k_new;           // [B, H_kv, d] the new token's key before rotation, or null
  const void* v_new;           // [B, H_kv, d] its value (with k_new)
  void* k_store;               // K_raw / V_raw: the new token's row is written at
  void* v_store;               //   index seq_raw[b] when that is below the capacity
  int32_t tok_slot0;           // partial slot of unit 0's new-token partial (then one per unit)
  // Paged ragged calls (page_table[0] or [1] set): seg[s].K / V are then
  // pools [num_pages[s], H_kv, 1 << page_shift, width] and sequence b's row
  // i of segment s lies in page page_table[s][b * table_width[s] + (i >> page_shift)]
  const int32_t* page_table[2];
  int32_t table_width[2];
  int32_t num_pages[2];
  int32_t page_shift;
  // Chunk calls: query tokens per sequence (q, out [B, Q, H_q, d], lse
  // [B, Q, H_q], k_new, v_new [B, Q, H_kv, d]); partials hold G * Q rows
  int32_t num_tokens;
  // ALiBi calls (alibi_slopes set): nothing is rotated and score j gets
  // -slope[h_q] * (q_pos - k_pos); beacon j at beacon_first + j *
  // beacon_stride, raw row t at q_pos - W + 1 + t
  const float* alibi_slopes;  // [H_q]
  int32_t beacon_first, beacon_stride;
};

// The full-width rebuild of the reconstruction paths: job 0 the keys
// (C_K, U_K), job 1 the values (C_V, U_V), both in one launch.
struct RebuildArgs {
  const void* C[2];  // [B, H_kv, N_b, r_job]
  const void* U[2];  // [H_kv, d, r_job]
  void* dst[2];      // [B, H_kv, N_b, d]
  int32_t rank[2];
  int32_t batch, num_kv_heads, num_beacons;
  const int32_t* pos;       // [N_b]: rotate key row j at pos[j] before rounding, or null
  double inv_freq_pow2[6];  // theta^(-2 * 2^k / d), as in AttnArgs (with pos)
};

// Host launchers (defined in the .hip files).  dtype: 0 fp32, 1 bf16.
// The attention kernel (bracketed by ev0/ev1 if set).
// a.chunks <= 0 lets the launcher pick the chunk count from the device's
// workgroup slots (CUs x resident workgroups of the chosen kernel).
hipError_t launch_attention(AttnArgs a, int dtype, hipStream_t s, hipEvent_t ev0,
                            hipEvent_t ev1);
// The ragged-batch attention kernel (one launch; see ragged_impl.h), over
// capacity-sized arrays or, with page tables in `a`, over page pools.
hipError_t launch_ragged(AttnArgs a, int dtype, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1);

// A chunk of query tokens per sequence over a ragged cache (one launch;
// bf16: chunk_impl.h, fp32 (dtype 0): chunk_f32_impl.h).
hipError_t launch_chunk(AttnArgs a, int dtype, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1);

// Chunks per unit: the count in [1, kMaxChunks] whose workgroups fill the
// device's slots best (no chunk under min_chunk_bytes).
int choose_chunks(int64_t units, int64_t unit_bytes, int64_t slots, int64_t min_chunk_bytes);
hipError_t launch_rebuild(const RebuildArgs& a, int dtype, hipStream_t s);

// Tile height (rows) a segment of the given widths is swept in.
int tile_rows(int dtype, int rk, int rv);

// SLIMKV_FLAG_CHECK_WORKSPACE: one small kernel, launched on `s` before a
// call's kernels, that finds every nonzero 32-bit word of ws[begin, end)
// (the counters and flags, which must start at zero), clears it, and sets
// bit 0 of ws word 0 when it found one.
hipError_t launch_workspace_check(uint32_t* ws, size_t begin, size_t end, hipStream_t s);

// Workgroup slots of the attention kernel that launch_attention would run
// for `a` (the device's CUs x resident workgroups of that kernel, at most
// kWgPerCu per CU), or <= 0 on a HIP error.  A device query, no launch.
int attention_slots(const AttnArgs& a, int dtype);

// The no-alloc entry point's device scratch (kNoAllocScratchBytes, one copy
// per device, kept until the process ends): its address on the current
// device (taken once per device with hipGetSymbolAddress), after launching
// on `s` a kernel that zeroes its first clear_bytes bytes.
hipError_t noalloc_scratch(size_t clear_bytes, hipStream_t s, void** ptr);

}  // namespace slimkv
