// chunk_impl.h -- a chunk of several query tokens per sequence (speculative
// decoding checks several drafted tokens at once; chunked prefill feeds a
// prompt a few tokens at a time) against the compressed cache, in one launch.
// Included by chunk.hip after sweep_impl.h, whose helpers it uses.
//
// What is computed is the attention of page "Can SlimKV compress KV cache
// jointly across tokens and features", section "Latent-space attention
// removes the rebuild step", for every query of the chunk: token t of
// sequence b sits at position q_pos[b] + t; each of its G query heads is
// rotated there (and projected into the KV head's latent key space for the
// beacon rows) and attends, under one softmax, over the sequence's live
// beacon rows, its live raw rows and the chunk's new tokens 0 .. t, whose
// keys are rotated at their own positions and rounded like cache rows.
// The chunk's tokens are then stored as raw rows w_b, w_b + 1, ... while
// the window has room.
//
// Mapping onto CDNA4 (bf16 caches):
//   * The M = G * Q <= 16 query rows of a (b, kv head) unit fill one MFMA
//     tile, so the value side is a dense contraction as well as the scores.
//   * Scores are taken transposed, S^T = K Q^T (cache rows on the MFMA's M
//     axis, query rows on N).  The output then holds, in lane (m, kg), query
//     row m's scores for cache rows 4kg .. 4kg+3 of each 16-row subtile --
//     after the exponent, exactly the B operand of v_mfma_f32_16x16x16_bf16
//     for O^T = V^T P^T.  The weights never leave registers (hi + lo bf16
//     terms, ~16 mantissa bits).  The value tile is transposed through LDS:
//     each wave stages its own tile row by row and reads 16-bit columns, rows
//     padded so that the four k-groups read different banks.
//   * O^T keeps query row m in lane m % 16's column, so the online-softmax
//     rescale is one multiply per register, and the latent sum O_lat^T is
//     already the B operand of the lift U_V O_lat^T, whose output lands in
//     the layout of the full-width sum.  Each wave lifts its own latent sum
//     after its last tile and parks one full-width sum.
//   * Work is shared out by tiles as in the ragged kernel (ragged_schedule,
//     ragged_piece_of); each workgroup writes one partial of M rows; the
//     unit's first workgroup also makes the chunk's tokens' partial before
//     its sweep, while its first tiles are in flight; the unit's last
//     workgroup merges them all.
#pragma once

namespace slimkv {

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

constexpr int kVPad = 4;  // value-tile row padding (elements)
// The largest padded value tile: 64 rows of r_V <= 32 (larger ranks have
// shorter tiles: 32 x (64 + 4), 16 x (128 + 4)).
constexpr int kVTileElems = 64 * (32 + kVPad);

struct alignas(16) ChunkShared {
  union {
    struct {
      union {
        uint16_t uk[64 * (kHeadDim + 2)];   // half of U_K's rows, padded (prologue)
        uint16_t vt[kWaves][kVTileElems];   // each wave's value tile (sweep)
        float tok[2][kChunkRows][kHeadDim];  // the chunk's keys (rotated, rounded) and values
                                             // (the unit's first workgroup, before its sweep)
      } x;
      float qrot[kChunkRows][kHeadDim];     // rotated query rows, pre-scaled
      float qlat[kChunkRows][kHeadDim];     // the same projected by U_K
    } s;
    uint16_t uv[kHeadDim * (kHeadDim + kVPad)];  // U_V, rows padded (the lift)
    float park[kWaves][kChunkRows][kHeadDim];  // each wave's full-width sums
  } u;
  float wml[kWaves][kChunkRows][2];  // each wave's (max, sum) per query row
  int is_last;
};

__device__ __forceinline__ float xor16_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ short bf16_bits(float x) {
  return __builtin_bit_cast(short, (__bf16)x);
}
// four fp32 values as hi + lo bf16 terms (as split_bf16x8)
__device__ __forceinline__ void split_bf16x4(const f32x4_t& x, s16x4_t& hi, s16x4_t& lo) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const __bf16 h = (__bf16)x[e];
    hi[e] = __builtin_bit_cast(short, h);
    lo[e] = bf16_bits(x[e] - (float)h);
  }
}

// Query rows of the chunk: row m is token m / G, head m % G of the unit.
// issue() requests the query and (latent beacons) both halves of U_K;
// finish() rotates the rows into sh.qrot (rows past M zero) and projects
// them, sh.qlat = qrot U_K, staging U_K in LDS half by half.
template <int NCH, bool ROTATE = true>
struct ChunkPrologue {
  static constexpr bool kLat = NCH > 0;
  static constexpr int kHalf = kHeadDim / 2;
  static constexpr int kPairs = kChunkRows * kHalf / kThreads;             // 4
  static constexpr int kWords = kLat ? 64 * 32 * NCH / 8 / kThreads : 1;  // per half, r_K <= 32 NCH
  u32x4_t qraw;  // query row tid / 16 (clamped to M - 1), columns 8 (tid % 16) .. +7
  int pos0;
  u32x4_t uk[2][kWords];

  __device__ __forceinline__ void issue(const AttnArgs& a, int b, int h, int M, int G) {
    const int tid = threadIdx.x;
    const int Q = a.num_tokens;
    {
      const int m = min(tid / 16, M - 1), c8 = tid & 15;
      const int t = m / G, g = m - t * G;
      const size_t base = (((size_t)b * Q + t) * a.num_q_heads + (size_t)h * G + g) * kHeadDim + 8 * c8;
      qraw = load16(static_cast<const uint16_t*>(a.q) + base);
    }
    pos0 = a.q_pos[b];
    if constexpr (kLat) {
      const int rk = a.rank_k, words = 64 * rk / 8;  // per half
      const char* U = static_cast<const char*>(a.U_K) + (size_t)h * kHeadDim * rk * 2;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int w = 0; w < kWords; ++w)
          uk[hf][w] = load16(U + ((size_t)hf * words + min(tid + kThreads * w, words - 1)) * 16);
    }
  }

  __device__ __forceinline__ void finish(const AttnArgs& a, ChunkShared& sh, int wave, int M,
                                         int G) const {
    const int tid = threadIdx.x, lane = tid & 63;
    const int n = lane & 15, kg = lane >> 4;
    const float sc = (float)a.score_scale;
    // the query rows into sh.qrot as they are (rotated in place below)
    {
      float* dst = &sh.u.s.qrot[tid / 16][8 * (tid & 15)];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dst[2 * e] = __uint_as_float(qraw[e] << 16);
        dst[2 * e + 1] = __uint_as_float(qraw[e] & 0xffff0000u);
      }
    }
    // the rotation depends on the token, not the head: each (token, pair)
    // angle is taken once, into a table in the space qlat takes later
    f32x2_t(*tab)[kHalf] = reinterpret_cast<f32x2_t(*)[kHalf]>(&sh.u.s.qlat[0][0]);
    if constexpr (ROTATE) {
      const int Q = a.num_tokens;
#pragma unroll
      for (int j = 0; j < kPairs; ++j) {
        const int t = wave + kWaves * j;  // token, pair `lane`
        if (t < Q) {
          float sn, cs;
          rope_sincos(a, pos0 + t, lane, sn, cs);
          tab[t][lane] = f32x2_t{sn, cs};
        }
      }
    }
    lds_barrier();
    // each (row, pair) is read and rewritten by one thread only
#pragma unroll
    for (int j = 0; j < kPairs; ++j) {
      const int p = tid + kThreads * j;  // < 16 * 64
      const int m = p / kHalf, i = p % kHalf;
      float r1 = 0.0f, r2 = 0.0f;
      if (m < M) {
        const float v1 = sh.u.s.qrot[m][i], v2 = sh.u.s.qrot[m][i + kHalf];
        if constexpr (ROTATE) {
          const f32x2_t t2 = tab[m / G][i];
          const float sn = t2[0], cs = t2[1];
          r1 = (v1 * cs - v2 * sn) * sc;
          r2 = (v2 * cs + v1 * sn) * sc;
        } else {  // an ALiBi backbone rotates nothing
          r1 = v1 * sc;
          r2 = v2 * sc;
        }
      }
      sh.u.s.qrot[m][i] = r1;
      sh.u.s.qrot[m][i + kHalf] = r2;
    }
    if constexpr (kLat) {
      // qlat[m][k] = sum_i qrot[m][i] U_K[i][k]: D[m][k] per 16-column tile
      // c0 = 16 (wave + 4 jt); A operand: query row n as hi + lo bf16
      // terms; B operand: U_K exact, lane (n, kg) takes rows 32c + 8kg ..
      // +7 of column c0 + n, from the staged half that holds them
      const int rk = a.rank_k, words = 64 * rk / 8, wpr = rk / 8, ustride = rk + 2;
      uint16_t* ul = sh.u.s.x.uk;
      f32x4_t d[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        if (hf == 1) lds_barrier();  // every wave is done with the first half
#pragma unroll
        for (int w = 0; w < kWords; ++w) {
          const int idx = tid + kThreads * w;
          if (idx < words) {
            const int row = idx / wpr, c8 = idx - row * wpr;
            uint32_t* dst = reinterpret_cast<uint32_t*>(ul + row * ustride + c8 * 8);
#pragma unroll
            for (int e = 0; e < 4; ++e) dst[e] = uk[hf][w][e];
          }
        }
        lds_barrier();  // (the first time also publishes qrot)
        bf16x8_t qh[2], ql[2];
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          const int i0 = 32 * (2 * hf + cc) + 8 * kg;
          const f32x4_t y0 = *reinterpret_cast<const f32x4_t*>(&sh.u.s.qrot[n][i0]);
          const f32x4_t y1 = *reinterpret_cast<const f32x4_t*>(&sh.u.s.qrot[n][i0 + 4]);
          const float x[8] = {y0[0], y0[1], y0[2], y0[3], y1[0], y1[1], y1[2], y1[3]};
          split_bf16x8(x, qh[cc], ql[cc]);
        }
#pragma unroll
        for (int jt = 0; jt < 2; ++jt) {
          const int c0 = 16 * (wave + kWaves * jt);
          if (c0 < rk) {
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) {
              u32x4_t bw;
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int i = 32 * cc + 8 * kg + 2 * e;  // row within the staged half
                bw[e] = (uint32_t)ul[i * ustride + c0 + n] |
                        ((uint32_t)ul[(i + 1) * ustride + c0 + n] << 16);
              }
              const bf16x8_t bv = __builtin_bit_cast(bf16x8_t, bw);
              d[jt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qh[cc], bv, d[jt], 0, 0, 0);
              d[jt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ql[cc], bv, d[jt], 0, 0, 0);
            }
          }
        }
      }
#pragma unroll
      for (int jt = 0; jt < 2; ++jt) {
        const int c0 = 16 * (wave + kWaves * jt);
        if (c0 < rk)
#pragma unroll
          for (int e = 0; e < 4; ++e) sh.u.s.qlat[4 * kg + e][c0 + n] = d[jt][e];
      }
    }
    lds_barrier();
  }
};

// The query of row n (lane % 16) as MFMA B operands for the scores: chunk c
// holds features 32c + 8kg .. +7 as hi + lo bf16 terms (zero past `width`).
template <int C>
__device__ __forceinline__ void chunk_query(const float (*src)[kHeadDim], int width, bf16x8_t (&hi)[C],
                                            bf16x8_t (&lo)[C]) {
  const int lane = threadIdx.x & 63, n = lane & 15, kg = lane >> 4;
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int k0 = 32 * c + 8 * kg;
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = k0 < width ? src[n][min(k0, kHeadDim - 8) + e] : 0.0f;
    split_bf16x8(x, hi[c], lo[c]);
  }
}

// A wave's softmax state and sums: lane (m, kg) holds query row m's running
// max (the same in its four k-group lanes), its share of the sum of
// weights, and O^T columns 16 cb + 4kg .. +3 of the latent (accb, NB
// blocks: r_V <= 16 NB) and full-width (accr) value sums.
template <int NB>
struct ChunkState {
  float m, l;
  f32x4_t accb[NB], accr[kHeadDim / 16];
};

// One tile of one segment: scores on the matrix cores, the next tile's keys
// requested, this tile's values staged in LDS and the next tile's values
// requested, then the online softmax and the value products.  t0: the
// tile's first row; rows: the segment's live rows; nchk: chunks carrying
// key features; width: value columns.  RAW: a raw tile, summed into accr
// (a rescale then applies to accb too); else a beacon tile, summed into
// accb (accr is not started: a wave's beacon tiles come first).
// ALIBI: score (row, query row m) gets s2 * (row * step - ofs), with s2 the
// query head's slope in log2 units and row * step - ofs = k_pos - (q_pos +
// t_m) for this lane's query row m (zero s2 on padding rows).  FETCH =
// false: the tile after this one is already in flight in other registers,
// so nothing is requested (jn, bv, rw, tail are unused).
template <int S, bool RAW, int NB, int SA, int SB, bool PG, bool ALIBI = false, bool FETCH = true>
__device__ __forceinline__ void chunk_tile(const SegView<S, true, PG>& sv, int t0, int nchk, int width,
                                           const bf16x8_t (&qh)[S], const bf16x8_t (&ql)[S],
                                           ChunkState<NB>& st, uint16_t* vt,
                                           const SegView<SA, true, PG>& bv,
                                           const SegView<SB, true, PG>& rw, int jn, int nbt,
                                           int total, const TailRows& tail, u32x4_t* kbuf,
                                           u32x4_t* vbuf, float s2 = 0.0f, int ofs = 0, int step = 0) {
  constexpr int SUB = SegView<S, true, PG>::kSub;
  constexpr int TR = SegView<S, true, PG>::kRows;
  constexpr int TRA = SegView<SA, true, PG>::kRows, TRB = SegView<SB, true, PG>::kRows;
  constexpr int VMAX = Traits<true>::kMaxLoads;
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, kg = lane >> 4;

  // scores S^T: lane (n = query row, kg) gets cache rows 16s + 4kg + e;
  // each subtile takes chunk c's hi then lo term, c ascending, with the
  // subtiles interleaved so that consecutive products are independent
  f32x4_t sc[SUB];
#pragma unroll
  for (int s = 0; s < SUB; ++s) sc[s] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int c = 0; c < S; ++c) {
    if (c < nchk) {
#pragma unroll
      for (int s = 0; s < SUB; ++s)
        sc[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kbuf[s * S + c]),
                                                        qh[c], sc[s], 0, 0, 0);
#pragma unroll
      for (int s = 0; s < SUB; ++s)
        sc[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kbuf[s * S + c]),
                                                        ql[c], sc[s], 0, 0, 0);
    }
  }
#pragma unroll
  for (int s = 0; s < SUB; ++s) {
    f32x4_t d = sc[s];
    if constexpr (ALIBI) {
#pragma unroll
      for (int e = 0; e < 4; ++e) d[e] = fmaf(s2, (float)((t0 + 16 * s + 4 * kg + e) * step - ofs), d[e]);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (t0 + 16 * s + 4 * kg + e >= sv.rows) d[e] = -INFINITY;
    sc[s] = d;
  }
  const bool ua = jn < nbt, ub = jn >= nbt && jn < total;
  const int pid = FETCH ? tile_page(bv, jn * TRA, ua, rw, (jn - nbt) * TRB, ub) : 0;
  if constexpr (FETCH) load_tile_keys<true>(bv, jn * TRA, ua, rw, (jn - nbt) * TRB, ub, tail, pid, kbuf);

  // this tile's values into the wave's LDS tile, row-major with padded rows
  const int pitch = width + kVPad;
#pragma unroll
  for (int i = 0; i < VMAX; ++i) {
    const int rt = i * sv.rpi + sv.vrow;
    if (sv.vact && rt < TR) {
      uint32_t* dst = reinterpret_cast<uint32_t*>(vt + rt * pitch + sv.vcc * 8);
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[e] = vbuf[i][e];
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if constexpr (FETCH) load_tile_values<true>(bv, jn * TRA, ua, rw, (jn - nbt) * TRB, ub, tail, pid, vbuf);

  // online softmax per query row (max over the row's 4 k-group lanes)
  float mx = sc[0][0];
#pragma unroll
  for (int s = 0; s < SUB; ++s)
#pragma unroll
    for (int e = 0; e < 4; ++e) mx = fmaxf(mx, sc[s][e]);
  mx = xor32_max(xor16_max(mx));
  const float mnew = fmaxf(st.m, mx);
  if (__builtin_amdgcn_ballot_w64(mnew > st.m) != 0) {
    const float alpha = __builtin_amdgcn_exp2f(st.m - mnew);
    st.l *= alpha;
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) st.accb[cb] *= alpha;
    if constexpr (RAW)
#pragma unroll
      for (int cb = 0; cb < kHeadDim / 16; ++cb) st.accr[cb] *= alpha;
    st.m = mnew;
  }
  s16x4_t ph[SUB], pl[SUB];
#pragma unroll
  for (int s = 0; s < SUB; ++s) {
    f32x4_t p;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      p[e] = __builtin_amdgcn_exp2f(sc[s][e] - st.m);
      st.l += p[e];
    }
    split_bf16x4(p, ph[s], pl[s]);
  }

  // O^T[col][m] += sum over rows V[row][col] P[m][row]: A operand lane
  // (n = column within the block, kg) holds rows 16s + 4kg .. +3
  // (each block takes subtile s's hi then lo term, s ascending; the blocks
  // are interleaved so that consecutive products are independent)
  constexpr int NA = RAW ? kHeadDim / 16 : NB;
  f32x4_t* acc = RAW ? st.accr : st.accb;
#pragma unroll
  for (int s = 0; s < SUB; ++s) {
    s16x4_t va[NA];
#pragma unroll
    for (int cb = 0; cb < NA; ++cb)
      if (16 * cb < width)
#pragma unroll
        for (int e = 0; e < 4; ++e) va[cb][e] = (short)vt[(16 * s + 4 * kg + e) * pitch + 16 * cb + n];
#pragma unroll
    for (int cb = 0; cb < NA; ++cb)
      if (16 * cb < width) acc[cb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va[cb], ph[s], acc[cb], 0, 0, 0);
#pragma unroll
    for (int cb = 0; cb < NA; ++cb)
      if (16 * cb < width) acc[cb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va[cb], pl[s], acc[cb], 0, 0, 0);
  }
  // the next tile overwrites the LDS tile: every lane has read it by now
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The chunk's tokens as an M-row partial, made by the unit's first
// workgroup between its prologue and its sweep, while its first tiles are in
// flight: query row m (token t, head g) over tokens 0 .. t, keys rotated at
// q_pos + u in fp64 and rounded once (the rows the cache keeps), scored
// against the rotated, pre-scaled query rows in LDS.  The partial --
// (max, sum) and the d sums per row -- goes to the unit's token slot
// (a.tok_slot0 + u) with device-coherent stores, for the merge; the
// tokens' rows are stored where the window has room (w + u < its
// capacity: no workgroup reads those rows in this call); PG: in the page
// the raw table gives for the row (ptab from rtab0; none if that id is out
// of range).  Thread (m, c8) owns 8 columns of row m (16 threads, one DPP
// row, per query row).  ALIBI: nothing is rotated (the keys are scored and
// stored as given) and query row m (token t) scoring token tk adds its
// head's slope times the distance tk - t (in log2 units).  BF16 / SH: the
// storage dtype and the kernel's LDS layout (fp32 caches have their own).
template <bool PG, bool ALIBI = false, bool BF16 = true, typename SH = ChunkShared>
__device__ __forceinline__ void chunk_token_partial(const AttnArgs& a, SH& sh, int u, int b,
                                                    int h, int wlive, int M, int G,
                                                    const int32_t* ptab, int rtab0) {
  const int tid = threadIdx.x;
  const int Q = a.num_tokens, Hkv = a.num_kv_heads;
  const int wcap = a.seg[1].rows;
  const int pos0 = a.q_pos[b];
  constexpr int kHalf = kHeadDim / 2;
  float (*kn)[kHeadDim] = sh.u.s.x.tok[0];
  float (*vn)[kHeadDim] = sh.u.s.x.tok[1];
  for (int p = tid; p < Q * kHalf; p += kThreads) {
    const int t = p / kHalf, i = p % kHalf;
    const size_t kb = (((size_t)b * Q + t) * Hkv + h) * kHeadDim;
    const uint32_t v1 = ld_bits<BF16>(a.v_new, kb + i), v2 = ld_bits<BF16>(a.v_new, kb + i + kHalf);
    uint32_t b1, b2;
    if constexpr (ALIBI) {
      b1 = ld_bits<BF16>(a.k_new, kb + i);
      b2 = ld_bits<BF16>(a.k_new, kb + i + kHalf);
    } else {
      const double k1 = (double)ld_elem<BF16>(a.k_new, kb + i);
      const double k2 = (double)ld_elem<BF16>(a.k_new, kb + i + kHalf);
      double s64, c64;
      sincos(rope_angle(a, pos0 + t, i), &s64, &c64);  // the reduced angle
      b1 = storage_bits_from_f64<BF16>(k1 * c64 - k2 * s64);
      b2 = storage_bits_from_f64<BF16>(k2 * c64 + k1 * s64);
    }
    kn[t][i] = bits_to_float<BF16>(b1);
    kn[t][i + kHalf] = bits_to_float<BF16>(b2);
    vn[t][i] = bits_to_float<BF16>(v1);
    vn[t][i + kHalf] = bits_to_float<BF16>(v2);
    if (wlive + t < wcap) {
      const int r = wlive + t;
      size_t row = ((size_t)u * wcap + r) * kHeadDim;
      bool store = true;
      if constexpr (PG) {
        const int sh_ = a.page_shift;
        const int pid = ptab[rtab0 + (r >> sh_)];
        store = (uint32_t)pid < (uint32_t)a.num_pages[1];
        row = ((((size_t)pid * a.num_kv_heads + h) << sh_) + (r & ((1 << sh_) - 1))) * kHeadDim;
      }
      if (store) {
        if constexpr (BF16) {
          uint16_t* kd = static_cast<uint16_t*>(a.k_store) + row;
          uint16_t* vd = static_cast<uint16_t*>(a.v_store) + row;
          kd[i] = (uint16_t)b1;
          kd[i + kHalf] = (uint16_t)b2;
          vd[i] = (uint16_t)v1;
          vd[i + kHalf] = (uint16_t)v2;
        } else {
          uint32_t* kd = static_cast<uint32_t*>(a.k_store) + row;
          uint32_t* vd = static_cast<uint32_t*>(a.v_store) + row;
          kd[i] = b1;
          kd[i + kHalf] = b2;
          vd[i] = v1;
          vd[i + kHalf] = v2;
        }
      }
    }
  }
  lds_barrier();
  const int mm = tid / 16, c8 = tid & 15;
  const int m = min(mm, M - 1), t = m / G;
  const float s2 = ALIBI ? a.alibi_slopes[h * G + m % G] * 1.4426950408889634f : 0.0f;
  float Mx = -INFINITY, L = 0.0f;
  f32x4_t acc[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
  for (int tk = 0; tk <= t; ++tk) {  // the 16 threads of a row share t
    float dot = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) dot += sh.u.s.qrot[m][8 * c8 + e] * kn[tk][8 * c8 + e];
    dot = row16_sum(dot);
    if constexpr (ALIBI) dot = fmaf(s2, (float)(tk - t), dot);
    const float mn = fmaxf(Mx, dot);
    const float a1 = __builtin_amdgcn_exp2f(Mx - mn), a2 = __builtin_amdgcn_exp2f(dot - mn);
    L = L * a1 + a2;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
      acc[hf] = acc[hf] * a1 + *reinterpret_cast<const f32x4_t*>(&vn[tk][8 * c8 + 4 * hf]) * a2;
    Mx = mn;
  }
  if (mm < M) {
    const size_t slot = (size_t)a.tok_slot0 + u;
    const __amdgpu_buffer_rsrc_t rs = coherent_rsrc(a.part_acc + slot * M * kHeadDim, M * kHeadDim * 4);
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, acc[hf]), rs,
                                             (m * kHeadDim + 8 * c8 + 4 * hf) * 4, 0, kCoherent);
    if (c8 == 0) {
      store_coherent(&a.part_ml[(slot * M + m) * 2], Mx);
      store_coherent(&a.part_ml[(slot * M + m) * 2 + 1], L);
    }
  }
  lds_barrier();  // every thread is done with the staged tokens (the sweep's value tiles alias them)
}

// The unit's last workgroup: fold the unit's nslots partials (slots slot0
// ..) and the chunk's tokens' partial (see chunk_token_partial; its loads
// are requested with the first partials', so the merge waits for memory
// once), then write out and lse.  Thread (m, c8) owns 8 columns of query
// row m.  A row with nothing to attend gets out 0 and lse -inf.
__device__ __forceinline__ void chunk_finish(const AttnArgs& a, int u, int b, int h, int slot0,
                                             int nslots, int M, int G) {
  const int tid = threadIdx.x;
  const int Q = a.num_tokens, Hq = a.num_q_heads;
  const int mm = tid / 16, c8 = tid & 15;  // query row, 8-column group
  const int m = min(mm, M - 1);
  const bool tok = a.k_new != nullptr;
  constexpr int kB = 8;
  uint32_t tml[2] = {0u, 0u};
  u32x4_t tacc[2] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};
  if (tok) {
    const size_t ts = (size_t)a.tok_slot0 + u;
    const __amdgpu_buffer_rsrc_t tm = coherent_rsrc(a.part_ml + ts * M * 2, M * 2 * 4);
    const __amdgpu_buffer_rsrc_t ta = coherent_rsrc(a.part_acc + ts * M * kHeadDim, M * kHeadDim * 4);
    tml[0] = __builtin_amdgcn_raw_buffer_load_b32(tm, m * 8, 0, kCoherent);
    tml[1] = __builtin_amdgcn_raw_buffer_load_b32(tm, m * 8 + 4, 0, kCoherent);
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
      tacc[hf] = __builtin_amdgcn_raw_buffer_load_b128(ta, (m * kHeadDim + 8 * c8 + 4 * hf) * 4, 0,
                                                      kCoherent);
  }
  const __amdgpu_buffer_rsrc_t rml =
      coherent_rsrc(a.part_ml + (size_t)slot0 * M * 2, (uint32_t)(nslots * M * 2 * 4));
  const __amdgpu_buffer_rsrc_t racc =
      coherent_rsrc(a.part_acc + (size_t)slot0 * M * kHeadDim, (uint32_t)(nslots * M * kHeadDim * 4));
  float Mx = -INFINITY, L = 0.0f;
  f32x4_t acc[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
  const auto fold = [&](uint32_t mbits, uint32_t lbits, const u32x4_t (&v)[2]) {
    const float ms = __uint_as_float(mbits), ls = __uint_as_float(lbits);
    const float mn = fmaxf(Mx, ms);
    if (mn != -INFINITY) {
      const float a1 = __builtin_amdgcn_exp2f(Mx - mn), a2 = __builtin_amdgcn_exp2f(ms - mn);
      L = L * a1 + ls * a2;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) acc[hf] = acc[hf] * a1 + __builtin_bit_cast(f32x4_t, v[hf]) * a2;
      Mx = mn;
    }
  };
  for (int s0 = 0; s0 < nslots; s0 += kB) {
    uint32_t mlw[kB][2];
    u32x4_t v[kB][2];
#pragma unroll
    for (int k = 0; k < kB; ++k) {
      const int s = min(s0 + k, nslots - 1);
      const int base = (s * M + m) * 8;
      mlw[k][0] = __builtin_amdgcn_raw_buffer_load_b32(rml, base, 0, kCoherent);
      mlw[k][1] = __builtin_amdgcn_raw_buffer_load_b32(rml, base + 4, 0, kCoherent);
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
        v[k][hf] = __builtin_amdgcn_raw_buffer_load_b128(
            racc, ((s * M + m) * kHeadDim + 8 * c8 + 4 * hf) * 4, 0, kCoherent);
    }
#pragma unroll
    for (int k = 0; k < kB; ++k)
      if (s0 + k < nslots) fold(mlw[k][0], mlw[k][1], v[k]);
  }
  if (tok) fold(tml[0], tml[1], tacc);
  if (mm < M) {
    const int t = m / G, g = m - t * G;
    const size_t row = ((size_t)b * Q + t) * Hq + (size_t)h * G + g;
    float* out = a.out + row * kHeadDim + 8 * c8;
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) *reinterpret_cast<f32x4_t*>(out + 4 * hf) = acc[hf] * inv;
    if (a.lse && c8 == 0)
      a.lse[row] = L > 0.0f ? (float)(0.69314718055994530942 * ((double)Mx + log2((double)L))) : -INFINITY;
  }
}

// The work of one workgroup of a chunk call: workgroup c of the k that share
// unit (b, h), as attend_unit, with the unit's live rows nbr, wr.  PG: the
// rows are paged; ptab (LDS) holds the unit's beacon page ids, then its raw
// page ids (those of its live rows and of the rows its tokens are stored in).
template <int NCH, bool PG, bool ALIBI = false>
__device__ __forceinline__ void chunk_unit(const AttnArgs& a, ChunkShared& sh, int unit, int b, int h,
                                           int c, int k, int nbr, int wr, int slot0,
                                           const int32_t* ptab) {
  constexpr bool BLAT = NCH > 0;
  constexpr int BN = BLAT ? NCH : 4;
  constexpr int TRB = SegView<BN, true, PG>::kRows, TRR = SegView<4, true, PG>::kRows;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, kg = lane >> 4;
  const int G = a.group, M = G * a.num_tokens;
  const int nwaves = kWaves * k;
  // the order in which tiles are dealt: the unit's first workgroup, which
  // also makes the chunk tokens' partial, comes last, so that it is the
  // one that gets a tile fewer when the unit's tiles do not divide evenly
  const int wu = kWaves * ((c + k - 1) % k) + wave;
  const int rk = BLAT ? a.seg[0].rk : 0, rv = BLAT ? a.seg[0].rv : 0;

  SegView<BN, true, PG> bv;
  SegView<4, true, PG> rw;
  int nbp = 0;  // the unit's beacon pages (paged)
  if constexpr (PG) {
    nbp = (nbr + (1 << a.page_shift) - 1) >> a.page_shift;
    bv.init_paged(a.seg[0].K, a.seg[0].V, a.page_shift, a.num_pages[0], nbr,
                  BLAT ? rk : kHeadDim, BLAT ? rv : kHeadDim, h, a.num_kv_heads, ptab, 0, lane);
    rw.init_paged(a.seg[1].K, a.seg[1].V, a.page_shift, a.num_pages[1], wr, kHeadDim, kHeadDim, h,
                  a.num_kv_heads, ptab, nbp, lane);
  } else {
    bv.init(a.seg[0].K, a.seg[0].V, a.seg[0].rows, nbr, BLAT ? rk : kHeadDim, BLAT ? rv : kHeadDim,
            unit, lane);
    rw.init(a.seg[1].K, a.seg[1].V, a.seg[1].rows, wr, kHeadDim, kHeadDim, unit, lane);
  }
  const int nbt = bv.ntiles, total = nbt + rw.ntiles;
  // Past its last tile a wave's load slots fetch its quarter of the head's
  // U_V for the lift (bytes 8192 wave .. +8191 of the 128 x r_V block: lanes
  // 4j .. 4j+3 take 256-byte block j through their four key slots, 64 bytes
  // apart, and block 16 + j through their value slots; bytes past the block
  // read as zeros), so it arrives with the wave's last tile.  Without
  // latent beacons the slots read a 16-byte window on q past its end.
  TailRows tail;
  if constexpr (BLAT) {
    tail.r = make_rsrc(static_cast<const char*>(a.U_V) + (size_t)h * kHeadDim * rv * 2,
                       (uint32_t)(kHeadDim * rv * 2));
    tail.klane = wave * 8192 + (lane & 3) * 16 + (lane >> 2) * 256;
    tail.vlane = tail.klane + 4096;
  } else {
    tail.r = make_rsrc(a.q, 16);
    tail.klane = tail.vlane = 64;
  }

  ChunkPrologue<NCH, !ALIBI> pro;
  pro.issue(a, b, h, M, G);
  // The wave's first tile, and -- when its first two tiles are both beacon
  // tiles -- its second, so that two tiles are in flight while the long
  // prologue runs (else the second set of slots reads the tail rows, and
  // goes unused).  The loads are issued on every path, so that the
  // prologue's waits do not depend on the branch.
  u32x4_t kbuf[Traits<true>::kMaxLoads], vbuf[Traits<true>::kMaxLoads];
  u32x4_t kbuf2[Traits<true>::kMaxLoads], vbuf2[Traits<true>::kMaxLoads];
  int j = wu;
  const bool two = BLAT && wu + nwaves < nbt;  // wave-uniform
  {
    const bool ub = j < nbt, ur = j >= nbt && j < total;
    const int pid = tile_page(bv, j * TRB, ub, rw, (j - nbt) * TRR, ur);
    load_tile_keys<true>(bv, j * TRB, ub, rw, (j - nbt) * TRR, ur, tail, pid, kbuf);
    load_tile_values<true>(bv, j * TRB, ub, rw, (j - nbt) * TRR, ur, tail, pid, vbuf);
    const int j2 = j + nwaves;
    const int pid2 = tile_page(bv, j2 * TRB, two, rw, 0, false);
    load_tile_keys<true>(bv, j2 * TRB, two, rw, 0, false, tail, pid2, kbuf2);
    load_tile_values<true>(bv, j2 * TRB, two, rw, 0, false, tail, pid2, vbuf2);
  }
  pro.finish(a, sh, wave, M, G);
  if (c == 0 && a.k_new)  // workgroup-uniform
    chunk_token_partial<PG, ALIBI>(a, sh, unit, b, h, wr, M, G, ptab, nbp);
  // ALiBi: this lane's query row m = n (token n / G, head n % G): its slope
  // in log2 units (zero on padding rows) and each segment's offset, so that
  // row * step - ofs = k_pos - q_pos - t (beacon j at first + j stride; raw
  // row i at q_pos - wr + i with new tokens, q_pos - wr + 1 + i without)
  float s2 = 0.0f;
  int bofs = 0, rofs = 0;
  if constexpr (ALIBI) {
    const int tm = n / G;
    s2 = n < M ? a.alibi_slopes[h * G + n % G] * 1.4426950408889634f : 0.0f;
    bofs = a.q_pos[b] - a.beacon_first + tm;
    rofs = (a.k_new ? wr : wr - 1) + tm;
  }

  constexpr int NB = BLAT ? 2 * BN : 1;  // latent sum blocks: r_V <= 32 NCH
  ChunkState<NB> st;
  st.m = -INFINITY;
  st.l = 0.0f;
#pragma unroll
  for (int cb = 0; cb < NB; ++cb) st.accb[cb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  uint16_t* vt = sh.u.s.x.vt[wave];
  // a wave's tiles come in order, beacon tiles first: one loop per segment,
  // so that only that segment's query operands and sums occupy registers
  if constexpr (BLAT) {
    bf16x8_t qlh[BN], qll[BN];
    chunk_query<BN>(sh.u.s.qlat, rk, qlh, qll);
    const int nchk = (rk + 31) / 32;
    if (two) {
      // the first tile requests the third; the second is already here
      chunk_tile<BN, false, NB, BN, 4, PG, ALIBI>(bv, j * TRB, nchk, rv, qlh, qll, st, vt, bv, rw,
                                                  j + 2 * nwaves, nbt, total, tail, kbuf, vbuf, s2,
                                                  bofs, a.beacon_stride);
      chunk_tile<BN, false, NB, BN, 4, PG, ALIBI, false>(bv, (j + nwaves) * TRB, nchk, rv, qlh, qll,
                                                         st, vt, bv, rw, 0, nbt, total, tail, kbuf2,
                                                         vbuf2, s2, bofs, a.beacon_stride);
      j += 2 * nwaves;
    }
    for (; j < nbt; j += nwaves)
      chunk_tile<BN, false, NB, BN, 4, PG, ALIBI>(bv, j * TRB, nchk, rv, qlh, qll, st, vt, bv, rw,
                                                  j + nwaves, nbt, total, tail, kbuf, vbuf, s2,
                                                  bofs, a.beacon_stride);
  }
#pragma unroll
  for (int cb = 0; cb < kHeadDim / 16; ++cb) st.accr[cb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  {
    bf16x8_t qrh[4], qrl[4];
    chunk_query<4>(sh.u.s.qrot, kHeadDim, qrh, qrl);
    for (; j < total; j += nwaves)
      chunk_tile<4, true, NB, BN, 4, PG, ALIBI>(rw, (j - nbt) * TRR, 4, kHeadDim, qrh, qrl, st, vt,
                                                bv, rw, j + nwaves, nbt, total, tail, kbuf, vbuf,
                                                s2, rofs, 1);
  }
  st.l = xor32_sum(xor16_sum(st.l));
  __builtin_amdgcn_s_setprio(2);  // from here on only the unit's finish: ahead of streaming waves
  lds_barrier();  // every wave is done with the query and value tiles (U_V and the park alias them)
  if constexpr (BLAT) {
    // U_V of head h staged in LDS (rows padded) from the waves' tail loads,
    // then each wave lifts its latent sum: accr^T[d][m] += sum_k U_V[d][k]
    // accb^T[k][m] per 16-row block of d; A operand lane (n, kg): U_V row
    // 16 db + n, columns 16 cb + 4kg .. +3; B operand: the latent sum as
    // hi + lo bf16 terms
    const int ncb = rv / 16, upitch = rv + kVPad, ubytes = kHeadDim * rv * 2;
#pragma unroll
    for (int i = 0; i < 2 * Traits<true>::kMaxLoads; ++i) {
      const int off = (i < 4 ? tail.klane : tail.vlane) + 64 * (i & 3);
      if (off < ubytes) {
        const int row = off / (2 * rv), col = (off - row * 2 * rv) / 2;
        uint32_t* dst = reinterpret_cast<uint32_t*>(sh.u.uv + row * upitch + col);
        const u32x4_t w = i < 4 ? kbuf[i] : vbuf[i - 4];
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[e] = w[e];
      }
    }
    lds_barrier();
    s16x4_t bh[NB], bl[NB];
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) split_bf16x4(st.accb[cb], bh[cb], bl[cb]);
    // each accumulator takes block cb's hi then lo term, cb ascending; the
    // d blocks are interleaved so that consecutive products are independent
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) {
      if (cb < ncb) {
        s16x4_t ua[kHeadDim / 16];
#pragma unroll
        for (int db = 0; db < kHeadDim / 16; ++db)
          ua[db] = *reinterpret_cast<const s16x4_t*>(sh.u.uv + (16 * db + n) * upitch + 16 * cb + 4 * kg);
#pragma unroll
        for (int db = 0; db < kHeadDim / 16; ++db)
          st.accr[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ua[db], bh[cb], st.accr[db], 0, 0, 0);
#pragma unroll
        for (int db = 0; db < kHeadDim / 16; ++db)
          st.accr[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ua[db], bl[cb], st.accr[db], 0, 0, 0);
      }
    }
    lds_barrier();  // every wave is done with U_V (the park aliases it)
  }
  if (kg == 0) {
    sh.wml[wave][n][0] = st.m;
    sh.wml[wave][n][1] = st.l;
  }
#pragma unroll
  for (int db = 0; db < kHeadDim / 16; ++db)
    *reinterpret_cast<f32x4_t*>(&sh.u.park[wave][n][16 * db + 4 * kg]) = st.accr[db];
  lds_barrier();

  // the workgroup's partial: M rows of (max, sum) and d sums
  const size_t slot = (size_t)slot0 + c;
  float* ml_out = a.part_ml + slot * M * 2;
  float* acc_out = a.part_acc + slot * M * kHeadDim;
  const __amdgpu_buffer_rsrc_t rs = coherent_rsrc(acc_out, (uint32_t)(M * kHeadDim * 4));
#pragma unroll
  for (int it = 0; it < kChunkRows * kHeadDim / 4 / kThreads; ++it) {
    const int idx = tid + kThreads * it;
    const int m = idx / (kHeadDim / 4), col = 4 * (idx % (kHeadDim / 4));
    if (m < M) {
      float Mx = sh.wml[0][m][0];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) Mx = fmaxf(Mx, sh.wml[w][m][0]);
      f32x4_t sum = {0.0f, 0.0f, 0.0f, 0.0f};
      float L = 0.0f;
      if (Mx != -INFINITY) {
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          const float wt = __builtin_amdgcn_exp2f(sh.wml[w][m][0] - Mx);
          sum += wt * *reinterpret_cast<const f32x4_t*>(&sh.u.park[w][m][col]);
          L += wt * sh.wml[w][m][1];
        }
      }
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, sum), rs, (m * kHeadDim + col) * 4,
                                             0, kCoherent);
      if (col == 0) {
        store_coherent(&ml_out[2 * m], Mx);
        store_coherent(&ml_out[2 * m + 1], L);
      }
    }
  }

  // the last workgroup of the unit merges (as attend_unit)
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) {
    const uint32_t done = __hip_atomic_fetch_add(&a.counters[(size_t)unit * kCounterStride], 1u,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sh.is_last = done == (uint32_t)(k - 1);
  }
  lds_barrier();
  if (!sh.is_last) return;
  if (tid < 2)
    __hip_atomic_store(&a.counters[(size_t)unit * kCounterStride + tid], 0u, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  chunk_finish(a, unit, b, h, slot0, k, M, G);
}

// One workgroup per piece, scheduled as the ragged kernel (ragged_schedule,
// ragged_piece_of): piece i of the batch is workgroup c of unit (b, h).  PG:
// the cache is paged; the workgroup first stages sequence b's page ids that
// it uses in LDS -- the pages of its live beacon rows, then of its live raw
// rows and of the rows that receive the chunk's tokens.
template <int NCH, bool PG, bool ALIBI = false>
__global__ __launch_bounds__(kThreads, kWgPerCu * kWaves / 4) void chunk_kernel(AttnArgs a) {
  constexpr int BN = NCH > 0 ? NCH : 4;
  constexpr int TRB = SegView<BN, true>::kRows, TRR = SegView<4, true>::kRows;
  __shared__ ChunkShared sh;
  __shared__ RaggedPick pick;
  __shared__ int32_t ptab[PG ? kMaxPageEntries : 1];
  const int tid = threadIdx.x;
  const int Hkv = a.num_kv_heads, P = a.chunks;
  const int pi = ragged_piece_of((int)blockIdx.x, P);
  ragged_schedule_wg<TRB, TRR>(a, pick, tid, P, pi);
  lds_barrier();
  const auto uni = [](int v) { return __builtin_amdgcn_readfirstlane(v); };
  if (pi >= uni(pick.total)) return;
  const int b = uni(pick.b), kb = uni(pick.k), first = uni(pick.first);
  const int h = (pi - first) / kb, c = pi - first - h * kb;
  const int nbr = uni(pick.nb), wr = uni(pick.w);
  if constexpr (PG) {
    // at most ceil(N_cap / rows) + ceil(W_cap / rows) <= kMaxPageEntries ids
    const int sh_ = a.page_shift, pm = (1 << sh_) - 1;
    const int nbp = (nbr + pm) >> sh_;
    const int wst = a.k_new ? min(wr + a.num_tokens, a.seg[1].rows) : wr;
    const int n = nbp + ((wst + pm) >> sh_);
    const int32_t* bt = a.page_table[0] + (size_t)b * a.table_width[0];
    const int32_t* rt = a.page_table[1] + (size_t)b * a.table_width[1];
    for (int i = tid; i < n; i += kThreads) ptab[i] = i < nbp ? bt[i] : rt[i - nbp];
    lds_barrier();
  }
  chunk_unit<NCH, PG, ALIBI>(a, sh, b * Hkv + h, b, h, c, kb, nbr, wr, first + h * kb, ptab);
}

}  // namespace slimkv
