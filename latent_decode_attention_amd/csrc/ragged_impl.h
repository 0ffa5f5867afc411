// ragged_impl.h -- decode attention over a ragged batch, with the decode
// step's new token (included by sweep_impl.h; instantiated per group size in
// sweep_g*.hip).
//
// What is computed is the latent decode attention of page "Can SlimKV
// compress KV cache jointly across tokens and features", section
// "Latent-space attention removes the rebuild step", in the setting of a
// serving decode step: every sequence b has its own number of live beacon
// rows and raw rows in capacity-sized arrays, and the step's new token --
// its key rotated at the query position, since the token attends to itself
// -- joins the raw rows.  When the raw window has room, the token's rotated
// key and its value are also written to the cache row after the live ones.
//
// Mapping onto CDNA4:
//   * Work is balanced over the grid by tiles, not by sequences: each unit
//     (b, kv head) gets a number of workgroups (pieces) in proportion to its
//     tiles -- as many as keep every piece at or below the smallest share
//     of tiles for which the pieces fit in the P workgroup slots, and at
//     least one.  Each workgroup then runs exactly what a
//     workgroup of the uniform kernel runs (attend_unit): the unit's tiles
//     dealt round-robin over all its pieces' waves, one partial per piece,
//     the last piece merging.
//   * Each workgroup recomputes the schedule from the lengths at its start:
//     one wave loads them, finds the share and finds its own piece, with
//     wave-wide sums on the VALU (no LDS tables, no shuffles through LDS).
//     Up to 64 sequences, the lanes test up to 64 candidate shares at once;
//     with at least as many units as slots, every unit is one piece and only
//     the workgroup's own sequence is read (see ragged_schedule).
//   * Pieces alternate between the CUs' first and second workgroup slots
//     and spread over the XCDs (see ragged_piece_of).
//   * The unit's first workgroup scores the new token and stores its row
//     in its prologue, while its first tile is in flight, and leaves a
//     one-row partial; the merge folds it in with the pieces' partials and
//     writes out and lse.  A unit without rows still gets its one piece,
//     which finds no tiles.
//   * Paged caches: rows sit in pages of at least 64 rows (a whole number
//     of tiles) from shared pools.  Each workgroup stages its sequence's
//     page ids in LDS once; a tile then costs one LDS read for its page id
//     and a descriptor over that page's live rows, so the tile loop and
//     the order of the arithmetic are those of the contiguous layout and
//     the results are bitwise the same.
#pragma once

namespace slimkv {

// The piece a workgroup runs: workgroup c of the k that share unit
// (b, h), c = (pi - first) % k, h = (pi - first) / k; sequence b has nb, w
// live rows; total pieces in the batch (a workgroup with pi >= total has
// nothing to do).
struct RaggedPick {
  int32_t b, first, k, nb, w, total;
  int32_t cnt[kWaves][64];  // the waves' partial piece counts per candidate share
};

// Wave-wide sums and maxima of integers on the VALU (DPP rotations within
// 16-lane rows, then permlane swaps across rows): no LDS round trips.
template <int CTRL>
__device__ __forceinline__ int dpp_i(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ int wave_sum_i(int x) {
  x += dpp_i<0x128>(x);
  x += dpp_i<0x124>(x);
  x += dpp_i<0x122>(x);
  x += dpp_i<0x121>(x);
  auto r = __builtin_amdgcn_permlane16_swap((uint32_t)x, (uint32_t)x, false, false);
  x = (int)(r[0] + r[1]);
  r = __builtin_amdgcn_permlane32_swap((uint32_t)x, (uint32_t)x, false, false);
  return (int)(r[0] + r[1]);
}
__device__ __forceinline__ int wave_max_i(int x) {
  x = max(x, dpp_i<0x128>(x));
  x = max(x, dpp_i<0x124>(x));
  x = max(x, dpp_i<0x122>(x));
  x = max(x, dpp_i<0x121>(x));
  auto r = __builtin_amdgcn_permlane16_swap((uint32_t)x, (uint32_t)x, false, false);
  x = max((int)r[0], (int)r[1]);
  r = __builtin_amdgcn_permlane32_swap((uint32_t)x, (uint32_t)x, false, false);
  return max((int)r[0], (int)r[1]);
}
// Inclusive prefix sum over the wave's lanes: shifts within 16-lane rows
// (lanes past a row's start read zero), then each row adds the totals of
// the rows before it.
__device__ __forceinline__ int wave_scan_i(int x, int lane) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);  // row_shr:8
  const int r0 = __builtin_amdgcn_readlane(x, 15), r1 = __builtin_amdgcn_readlane(x, 31);
  const int r2 = __builtin_amdgcn_readlane(x, 47);
  const int row = lane >> 4;
  return x + (row > 0 ? r0 : 0) + (row > 1 ? r1 : 0) + (row > 2 ? r2 : 0);
}

// Run by one wave: live rows clamped to [0, capacity], the tiles t of each
// of a sequence's units, and the pieces (workgroups) per unit
// k = clamp(ceil(t / L), 1, kMaxChunks) for the smallest share L (tiles per
// piece) at which all pieces fit in the P workgroup slots -- so the busiest
// workgroup has as few tiles as the slots allow -- or one piece per unit if
// even that does not fit.  A unit without rows still gets its piece.  The
// pieces are numbered sequence by sequence (lane L takes a run of
// consecutive sequences; every load is requested before any is used), and
// the lane whose sequence holds piece pi writes it to `pick`.
template <int TRB, int TRR>
__device__ __forceinline__ void ragged_schedule(const AttnArgs& a, RaggedPick& pick, int lane, int P,
                                                int pi) {
  constexpr int kPer = kMaxRaggedBatch / 64;
  const int B = a.batch, ncap = a.seg[0].rows, wcap = a.seg[1].rows, Hkv = a.num_kv_heads;
  // Every per-lane loop below stops after `per` (wave-uniform) iterations:
  // unrolled to kPer with only a guard, the divisions of all kPer
  // iterations would run under an execution mask at every step of the search.
  const int per = (B + 63) / 64;
  const int b0 = lane * per;
  const int units = B * Hkv;
  if (units >= P) {
    // As many units as slots or more: whatever the lengths, every unit gets
    // one piece (the search below would end at a share no unit exceeds), so
    // piece pi is unit pi and only its sequence's lengths are needed.
    if (lane == 0) {
      const int b = min(pi / Hkv, B - 1);
      const int nb = a.seq_beacons ? a.seq_beacons[b] : ncap;
      const int w = a.seq_raw ? a.seq_raw[b] : wcap;
      pick.b = b;
      pick.first = b * Hkv;
      pick.k = 1;
      pick.nb = min(max(nb, 0), ncap);
      pick.w = min(max(w, 0), wcap);
      pick.total = units;
    }
    return;
  }
  int nbv[kPer], wv[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    if (k == per) break;
    const int b = min(b0 + k, B - 1);
    nbv[k] = a.seq_beacons ? a.seq_beacons[b] : ncap;
    wv[k] = a.seq_raw ? a.seq_raw[b] : wcap;
  }
  int tiles[kPer];
  int sum = 0, tmax = 0;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    if (k == per) break;
    nbv[k] = min(max(nbv[k], 0), ncap);
    wv[k] = min(max(wv[k], 0), wcap);
    const bool mine = b0 + k < B;
    tiles[k] = mine ? (nbv[k] + TRB - 1) / TRB + (wv[k] + TRR - 1) / TRR : -1;  // -1: not a sequence
    if (mine) {
      sum += tiles[k];
      tmax = max(tmax, tiles[k]);
    }
  }
  const auto pieces = [](int t, int L) { return t < 0 ? 0 : min(max((t + L - 1) / L, 1), kMaxChunks); };
  // pieces of the whole batch at share L
  const auto count = [&](int L) {
    int c = 0;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      if (k == per) break;
      c += pieces(tiles[k], L);
    }
    return wave_sum_i(c) * Hkv;
  };
  const int T = wave_sum_i(sum) * Hkv;  // the host checks that the batch's tiles fit in int32
  tmax = wave_max_i(tmax);
  // L >= T / P, as P pieces must hold T tiles; and L = T / (P - units)
  // always fits (sum of ceil(t / L) <= T / L + units), which bounds the
  // search when the slots outnumber the units
  int lo = max(1, (T + P - 1) / P), hi = max(lo, tmax);
  if (P > units) hi = min(hi, max(lo, (T + (P - units) - 1) / (P - units)));
  if (per == 1 && hi - lo < 64 && tmax < (1 << 23)) {
    // Every sequence in a lane of its own and fewer than 64 candidates: lane
    // j counts the pieces at share lo + j over the whole batch, all lanes
    // at once, and the smallest share that fits wins (as the search below
    // would find).  The quotient is formed from the reciprocal, clamped to
    // 65 and corrected by one either way (24-bit products): exact wherever
    // the clamp to kMaxChunks does not hide it, for t and L below 2^23.
    // Four sequences per pass keep four independent chains in flight.
    const int Lc = lo + lane;
    const float rc = __builtin_amdgcn_rcpf((float)Lc);
    const auto pieces_at = [&](int t) {
      int q = min((int)__builtin_ceilf((float)t * rc), kMaxChunks + 1);
      if (__mul24(q - 1, Lc) >= t) --q;
      if (__mul24(q, Lc) < t) ++q;
      return min(max(q, 1), kMaxChunks);
    };
    int c = 0;
    for (int s = 0; s < B; s += 4) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int p = pieces_at(__builtin_amdgcn_readlane(tiles[0], min(s + i, 63)));
        c += s + i < B ? p : 0;
      }
    }
    const uint64_t fits = __builtin_amdgcn_ballot_w64(c * Hkv <= P && Lc <= hi);
    if (fits) hi = lo + __builtin_ctzll(fits);
  } else if (count(lo) <= P) {
    hi = lo;
  } else if (count(hi) <= P) {  // the smallest L in (lo, hi] with count(L) <= P (count falls with L)
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (count(mid) <= P) hi = mid; else lo = mid;
    }
  }
  const int L = hi;
  int pk[kPer];
  int psum = 0;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    if (k == per) break;
    pk[k] = pieces(tiles[k], L);
    psum += pk[k] * Hkv;
  }
  const int incl = wave_scan_i(psum, lane);
  int run = incl - psum;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    if (k == per) break;
    if (pk[k] > 0 && pi >= run && pi < run + pk[k] * Hkv) {
      pick.b = b0 + k;
      pick.first = run;
      pick.k = pk[k];
      pick.nb = nbv[k];
      pick.w = wv[k];
    }
    run += pk[k] * Hkv;
  }
  if (lane == 63) pick.total = incl;
}

// ragged_schedule run by the whole workgroup (tid = threadIdx.x): up to 64
// sequences with fewer than 64 candidate shares, the four waves count the
// pieces at every candidate over a quarter of the sequences each (wave w
// takes sequences w, w + 4, ...) and add their counts through LDS, so the
// search takes a quarter of the steps; wave 0 then numbers the pieces.
// Every other case is ragged_schedule on wave 0.  The share found, and so
// the pick, is the same.  The caller's LDS barrier follows.
template <int TRB, int TRR>
__device__ __forceinline__ void ragged_schedule_wg(const AttnArgs& a, RaggedPick& pick, int tid, int P,
                                                   int pi) {
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int B = a.batch, ncap = a.seg[0].rows, wcap = a.seg[1].rows, Hkv = a.num_kv_heads;
  const int units = B * Hkv;
  // workgroup-uniform throughout: every wave sees the same lengths
  bool fast = units < P && B <= 64;
  int nb = 0, w = 0, tiles = -1, lo = 1, hi = 1;
  const bool mine = lane < B;
  if (fast) {
    // lane b holds sequence b (every wave loads the lengths)
    const int bl = min(lane, B - 1);
    nb = a.seq_beacons ? a.seq_beacons[bl] : ncap;
    w = a.seq_raw ? a.seq_raw[bl] : wcap;
    nb = min(max(nb, 0), ncap);
    w = min(max(w, 0), wcap);
    tiles = mine ? (nb + TRB - 1) / TRB + (w + TRR - 1) / TRR : -1;
    const int T = wave_sum_i(mine ? tiles : 0) * Hkv;
    const int tmax = wave_max_i(mine ? tiles : 0);
    lo = max(1, (T + P - 1) / P);
    hi = max(lo, tmax);
    if (P > units) hi = min(hi, max(lo, (T + (P - units) - 1) / (P - units)));
    fast = hi - lo < 64 && tmax < (1 << 23);
  }
  if (!fast) {
    if (wave == 0) ragged_schedule<TRB, TRR>(a, pick, lane, P, pi);
    return;
  }
  // ceil(t / L) for t, L below 2^23, from the reciprocal, clamped to 65 and
  // corrected by one either way (as in ragged_schedule), then clamped to
  // [1, kMaxChunks]
  const auto pieces_at = [](int t, int L, float rc) {
    int q = min((int)__builtin_ceilf((float)t * rc), kMaxChunks + 1);
    if (__mul24(q - 1, L) >= t) --q;
    if (__mul24(q, L) < t) ++q;
    return min(max(q, 1), kMaxChunks);
  };
  // lane j: pieces at share lo + j over this wave's sequences
  const int Lc = lo + lane;
  const float rc = __builtin_amdgcn_rcpf((float)Lc);
  int c = 0;
  for (int s = wave; s < B; s += kWaves) c += pieces_at(__builtin_amdgcn_readlane(tiles, s), Lc, rc);
  pick.cnt[wave][lane] = c;
  lds_barrier();
  if (wave != 0) return;
  c = pick.cnt[0][lane];
#pragma unroll
  for (int v = 1; v < kWaves; ++v) c += pick.cnt[v][lane];
  const uint64_t fits = __builtin_amdgcn_ballot_w64(c * Hkv <= P && Lc <= hi);
  const int L = fits ? lo + __builtin_ctzll(fits) : hi;
  const int pk = mine ? pieces_at(tiles, L, __builtin_amdgcn_rcpf((float)L)) : 0;
  const int psum = pk * Hkv;
  const int incl = wave_scan_i(psum, lane);
  const int run = incl - psum;
  if (pk > 0 && pi >= run && pi < run + psum) {
    pick.b = lane;
    pick.first = run;
    pick.k = pk;
    pick.nb = nb;
    pick.w = w;
  }
  if (lane == 63) pick.total = incl;
}

// Piece (workgroup slot) of block blk among the first P blocks, which take
// a CU's first and second workgroup slots in turn: the first half of them
// the even pieces, the second half the odd ones shifted by four blocks, so
// a unit's neighbouring pieces run in both slots and on different XCDs.
// Blocks from P on keep their index.
__device__ __forceinline__ int ragged_piece_of(int blk, int P) {
  if (blk >= P || (P & 1)) return blk;
  const int half = P >> 1;
  if (blk < half) return 2 * blk;
  int m = (blk - half - 4) % half;
  if (m < 0) m += half;
  return 2 * m + 1;
}

// One workgroup per piece: the grid is a.chunks (the device's workgroup
// slots, P), or one block per unit if the units are more; that is enough
// for every piece, and blocks past the last piece return at once.  Piece i of the
// batch is workgroup c of unit (b, h) as in the uniform kernel, with the
// unit's live rows and its k[b] workgroups.  PG: the cache is paged; the
// workgroup first stages sequence b's page ids that it uses -- the pages
// of its live beacon rows, then of its live raw rows and of the row that
// receives the new token -- in LDS.
template <int G, int NCH, bool BF16, bool PG, bool ALIBI = false>
__global__ __launch_bounds__(kThreads, kWgPerCu * kWaves / 4) void ragged_kernel(AttnArgs a) {
  constexpr bool BLAT = NCH > 0;
  constexpr int kFullNch = BF16 ? 4 : 8;
  constexpr int BN = BLAT ? NCH : kFullNch;
  constexpr int TRB = SegView<BN, BF16>::kRows, TRR = SegView<kFullNch, BF16>::kRows;
  __shared__ AttnShared sh;
  __shared__ RaggedPick pick;
  __shared__ int32_t ptab[PG ? kMaxPageEntries : 1];
  const int tid = threadIdx.x;
  const int Hkv = a.num_kv_heads, P = a.chunks;
  const int pi = ragged_piece_of((int)blockIdx.x, P);
  ragged_schedule_wg<TRB, TRR>(a, pick, tid, P, pi);
  lds_barrier();
  // values read back from LDS are the same in every lane: readfirstlane
  // keeps what derives from them (addresses, descriptors) in scalar registers
  const auto uni = [](int v) { return __builtin_amdgcn_readfirstlane(v); };
  if (pi >= uni(pick.total)) return;  // workgroup-uniform
  const int b = uni(pick.b), kb = uni(pick.k), first = uni(pick.first);
  const int h = (pi - first) / kb, c = pi - first - h * kb;
  const int nbr = uni(pick.nb), wr = uni(pick.w);
  if constexpr (PG) {
    // at most ceil(N_cap / rows) + ceil(W_cap / rows) <= kMaxPageEntries ids
    const int sh_ = a.page_shift, pm = (1 << sh_) - 1;
    const int nbp = (nbr + pm) >> sh_;
    const int wst = (a.k_new && wr < a.seg[1].rows) ? wr + 1 : wr;
    const int n = nbp + ((wst + pm) >> sh_);
    const int32_t* bt = a.page_table[0] + (size_t)b * a.table_width[0];
    const int32_t* rt = a.page_table[1] + (size_t)b * a.table_width[1];
    for (int i = tid; i < n; i += kThreads) ptab[i] = i < nbp ? bt[i] : rt[i - nbp];
    lds_barrier();
  }
  attend_unit<G, NCH, BF16, true, PG, ALIBI>(a, sh, b * Hkv + h, b, h, c, kb, nbr, wr, first + h * kb,
                                             ptab);
}

// Launch for group size G; nch as for launch_attention_group.
template <int G, bool PG, bool AL>
const void* ragged_kernel_for(int dtype, int nch) {
  if (dtype == 0)
    return nch == 0 ? reinterpret_cast<const void*>(&ragged_kernel<G, 0, false, PG, AL>)
                    : reinterpret_cast<const void*>(&ragged_kernel<G, 8, false, PG, AL>);
  switch (nch) {
    case 0: return reinterpret_cast<const void*>(&ragged_kernel<G, 0, true, PG, AL>);
    case 1: return reinterpret_cast<const void*>(&ragged_kernel<G, 1, true, PG, AL>);
    case 2: return reinterpret_cast<const void*>(&ragged_kernel<G, 2, true, PG, AL>);
    case 3: return reinterpret_cast<const void*>(&ragged_kernel<G, 3, true, PG, AL>);
    default: return reinterpret_cast<const void*>(&ragged_kernel<G, 4, true, PG, AL>);
  }
}

// P = a.chunks (> 0: as given; <= 0: the device's workgroup slots), at most
// max_wgs; the grid adds one block per unit (at most max_wgs in all)
template <int G>
hipError_t launch_ragged_group(AttnArgs a, int dtype, int nch, int64_t max_wgs, hipStream_t s,
                               hipEvent_t ev0, hipEvent_t ev1) {
  const bool paged = a.page_table[0] != nullptr || a.page_table[1] != nullptr;
  const bool alibi = a.alibi_slopes != nullptr;
  const void* kfn = paged ? (alibi ? ragged_kernel_for<G, true, true>(dtype, nch)
                                   : ragged_kernel_for<G, true, false>(dtype, nch))
                          : (alibi ? ragged_kernel_for<G, false, true>(dtype, nch)
                                   : ragged_kernel_for<G, false, false>(dtype, nch));
  int64_t P = a.chunks;
  if (P <= 0) {
    P = device_slots(kfn);
    if (P <= 0) return hipErrorInvalidDeviceFunction;
  }
  P = std::min<int64_t>(P, max_wgs);
  a.chunks = (int32_t)P;
  // pieces: at most P when the slots outnumber the units (the share search
  // then always fits them), else one per unit
  const int64_t units = (int64_t)a.batch * a.num_kv_heads;
  const dim3 grid((unsigned)std::min<int64_t>(std::max<int64_t>(P, units), max_wgs)), block(kThreads);
  if (ev0) {
    const hipError_t err = hipEventRecord(ev0, s);
    if (err != hipSuccess) return err;
  }
  void* args[] = {&a};
  hipError_t err = hipLaunchKernel(kfn, grid, block, args, 0, s);
  if (err == hipSuccess) err = hipGetLastError();
  if (err == hipSuccess && ev1) return hipEventRecord(ev1, s);
  return err;
}

}  // namespace slimkv
