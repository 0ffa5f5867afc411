// internal.h -- launch plan shared by the host API (api.cpp) and the HIP
// kernels.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace slimkv {

constexpr int kHeadDim = 128;
constexpr int kWaves = 4;              // waves per sweep workgroup
constexpr int kThreads = 64 * kWaves;  // sweep / combine workgroup size
constexpr int kMaxGroup = 8;           // query heads per KV head (G)
constexpr int kMaxSplits = 4096;       // row chunks per segment per unit

enum SegKind : int32_t {
  kSegLatent = 0,  // beacon rows: keys of width r_K scored with the latent
                   // query, values of width r_V summed in latent space
  kSegFull = 1,    // full-width rows (raw window, rebuilt beacons, full KV)
};

// One run of rows that every (b, kv head) unit owns, e.g. its N_b beacons.
struct Segment {
  const void* K;      // [B, H_kv, rows, rk]
  const void* V;      // [B, H_kv, rows, rv]
  int32_t kind;       // SegKind
  int32_t rows;       // rows per unit
  int32_t rk, rv;     // row widths in elements (d for kSegFull)
  int32_t splits;     // chunks per unit
  int32_t chunk_rows; // rows per chunk (multiple of the tile height)
};

// Everything the sweep and combine kernels read.
struct SweepArgs {
  Segment seg[2];
  int32_t nseg;
  int32_t batch, num_q_heads, num_kv_heads, group;
  int32_t splits_total;       // seg[0].splits + seg[1].splits
  const float* q_lat;         // [B, H_q, r_K] latent query, pre-scaled
  const float* q_rot;         // [B, H_q, d] rotated query, pre-scaled
  float* part_ml;             // [units, splits_total, G, 2]  (max, sum)
  float* part_acc;            // [units, splits_total, G, d]  weighted values
};

struct PrologueArgs {
  const void* q;              // [B, H_q, d]
  const int32_t* q_pos;       // [B]
  const void* U_K;            // [H_kv, d, r_K] or null
  int32_t batch, num_q_heads, num_kv_heads, group, rank_k;
  double rope_theta;
  double score_scale;         // scale * log2(e): scores come out in log2 units
  float* q_rot;               // out: [B, H_q, d]
  float* q_lat;               // out: [B, H_q, r_K] or null
};

struct CombineArgs {
  const float* part_ml;
  const float* part_acc;
  const void* U_V;            // [H_kv, d, r_V] or null (no latent segment)
  int32_t batch, num_q_heads, num_kv_heads, group, rank_v;
  int32_t splits_total;
  int32_t latent_splits;      // leading splits that hold latent sums (r_V wide)
  float* out;                 // [B, H_q, d]
  float* lse;                 // [B, H_q] or null
};

struct RebuildArgs {
  const void* C;              // [B, H_kv, N_b, r]
  const void* U;              // [H_kv, d, r]
  void* dst;                  // [B, H_kv, N_b, d]
  int32_t batch, num_kv_heads, num_beacons, rank;
};

// Host launchers (defined in the .hip files).  dtype: 0 fp32, 1 bf16.
hipError_t launch_prologue(const PrologueArgs& a, int dtype, hipStream_t s);
hipError_t launch_sweep(const SweepArgs& a, int dtype, hipStream_t s);
hipError_t launch_combine(const CombineArgs& a, int dtype, hipStream_t s);
hipError_t launch_rebuild(const RebuildArgs& a, int dtype, hipStream_t s);

// Tile height (rows) a segment of the given widths is swept in.
int tile_rows(int dtype, int rk, int rv);

}  // namespace slimkv
