/*
 * slimkv.h -- C ABI of libslimkv.so: SlimKV reconstruction-free latent
 * decode attention on AMD Instinct MI355X (gfx950).
 *
 * The operation (page "Can SlimKV compress KV cache jointly across tokens
 * and features", section "Latent-space attention removes the rebuild step";
 * also the abstract on page "SlimKV: Joint Token-Feature KV Cache
 * Compression with Reconstruction-Free Beacon Attention"):
 *
 *   A decode step attends over a cache compressed along tokens and
 *   features.  Older context lives in N_b beacon rows held as low-rank
 *   latents C_K (rank r_K) and C_V (rank r_V); their keys are trained
 *   without rotary position, so they are stored and used unrotated.  The W
 *   most recent tokens stay as raw rows K_raw, V_raw at the full head
 *   dimension d, their keys rotated at their own positions.  The query is
 *   always rotated.  After grouped-query grouping, each query head h_q
 *   (KV head h = h_q / G, G = H_q / H_kv) is projected into its KV head's
 *   latent key space, (q' U_K), scored against C_K and, at full width,
 *   against K_raw, with one softmax over all N_b + W scores.  Beacon values
 *   are summed in latent form, (A C_V), and lifted once by U_V.  Beacon keys
 *   are never rebuilt at full dimension.
 *
 *   Per query head, with q' = RoPE(q, q_pos) (rotate-half pairs (i, i+d/2),
 *   angle q_pos * theta^(-2i/d)):
 *     s_j       = scale * (U_K^T q') . C_K[j]        j < N_b
 *     s_{N_b+t} = scale * q' . K_raw[t]              t < W
 *     a         = softmax(s)
 *     out       = U_V (sum_j a_j C_V[j]) + sum_t a_{N_b+t} V_raw[t]
 *     lse       = log(sum_j exp(s_j))                (natural log)
 *
 * Memory and threading rules common to every entry point:
 *   - Tensor arguments are DEVICE pointers to contiguous row-major arrays
 *     in the layouts listed below, 16-byte aligned.  The problem struct is
 *     host memory.
 *   - The caller owns every buffer; the library never allocates, frees or
 *     synchronises, and keeps no state between calls.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL is the null
 *     stream).  Buffers must stay valid until the stream has run the call.
 *   - Inputs are read only.  out, lse and the workspace must not overlap
 *     any input or each other.
 *   - Every argument check happens before any HIP call.  On error nothing
 *     is launched, outputs are untouched, and a status is returned; the
 *     library never aborts or throws across this ABI.  slimkv_last_error()
 *     then describes the failed check (per calling thread).
 *   - The workspace is scratch of slimkv_workspace_bytes() bytes.  It must
 *     be zero-filled once before its first use; each completed call leaves
 *     it fit for the next.  Calls that share a workspace must be ordered on
 *     one stream: calls running at the same time on different streams must
 *     not share one (their counters would mix).  SLIMKV_FLAG_CHECK_WORKSPACE
 *     checks the counters before a call.
 *   - bf16 means the upper 16 bits of an IEEE-754 binary32 (round to
 *     nearest even is the caller's business).
 */
#ifndef SLIMKV_H
#define SLIMKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SLIMKV_ABI_VERSION 9

typedef enum slimkv_status {
  SLIMKV_OK = 0,
  SLIMKV_ERR_NULL = 1,        /* a required pointer is NULL                 */
  SLIMKV_ERR_SHAPE = 2,       /* inconsistent or out-of-range sizes         */
  SLIMKV_ERR_UNSUPPORTED = 3, /* valid, but outside what the kernels cover  */
  SLIMKV_ERR_WORKSPACE = 4,   /* workspace smaller than required            */
  SLIMKV_ERR_ALIGN = 5,       /* a device pointer is not 16-byte aligned    */
  SLIMKV_ERR_ALIAS = 6,       /* an output overlaps an input or another one */
  SLIMKV_ERR_HIP = 7          /* a HIP launch failed                        */
} slimkv_status;

typedef enum slimkv_dtype {
  SLIMKV_FP32 = 0, /* IEEE binary32 */
  SLIMKV_BF16 = 1  /* bfloat16      */
} slimkv_dtype;

typedef enum slimkv_op {
  SLIMKV_OP_LATENT = 0,      /* slimkv_decode_attn      */
  SLIMKV_OP_RECONSTRUCT = 1, /* slimkv_reconstruct_attn */
  SLIMKV_OP_FULL_KV = 2,     /* full_kv_attn            */
  SLIMKV_OP_LATENT_RAGGED = 3 /* slimkv_decode_attn_ragged, _paged */
} slimkv_op;

/* Shape of one layer's call (56 bytes, no implicit padding). */
typedef struct slimkv_problem {
  int32_t batch;        /* B >= 1                                            */
  int32_t num_q_heads;  /* H_q, a multiple of H_kv; G = H_q / H_kv <= 8      */
  int32_t num_kv_heads; /* H_kv >= 1                                         */
  int32_t head_dim;     /* d; must be 128                                    */
  int32_t num_beacons;  /* N_b >= 0 beacon rows per (b, kv head), <= 2^22    */
  int32_t rank_k;       /* r_K: multiple of 16 in [16, 128] when N_b > 0     */
  int32_t rank_v;       /* r_V: multiple of 16 in [16, 128] when N_b > 0     */
  int32_t raw_window;   /* W >= 0 raw rows per (b, kv head), <= 2^22;
                           N_b + W >= 1                                      */
  float scale;          /* softmax scale, finite and > 0 (e.g. 1/sqrt(d))   */
  int32_t dtype;        /* slimkv_dtype of q, U_K, U_V, C_K, C_V, K, V       */
  double rope_theta;    /* rotary base, finite and > 1                       */
  int32_t num_splits;   /* 0: library picks; > 0: workgroups that share each
                           (b, kv head)'s rows (at most 64)                 */
  int32_t flags;        /* SLIMKV_FLAG_* bits below; other bits 0            */
} slimkv_problem;

/*
 * Row scheduling.  By default the tiles of a (b, kv head)'s rows are dealt
 * round-robin over its workgroups' waves in a fixed order: repeated calls
 * on the same device and problem give bitwise equal out and lse.  With
 * SLIMKV_FLAG_DYNAMIC_TILES the waves take tiles from a shared counter
 * instead, so faster ones take more (useful when other work shares the
 * GPU); the order in which rows are summed then depends on timing, and
 * repeated calls agree only to rounding (well inside the documented
 * tolerances).
 */
#define SLIMKV_FLAG_DYNAMIC_TILES 1

/*
 * Workspace check (debugging).  With SLIMKV_FLAG_CHECK_WORKSPACE a call
 * first runs a small kernel that checks that the workspace's counters and
 * flags are zero, as the contract requires (a workspace that was never
 * zero-filled, one left by a call that did not run to its end, or one used
 * by calls on two streams at once breaks it).  Nonzero words are cleared,
 * so the call's results are still right, and bit 0 of the workspace's
 * status word is set; slimkv_workspace_status reads it.  The check costs
 * one extra launch per call.  Accepted by every entry point (ragged, paged
 * and chunk calls take no other flag); the no-alloc entry point clears its
 * scratch on every call, so there the flag has nothing to check.
 */
#define SLIMKV_FLAG_CHECK_WORKSPACE 2

/*
 * Workspace bytes the given op needs for this problem, or 0 if the problem
 * is invalid (the entry point would return an error; slimkv_last_error()
 * says why).  Pure host arithmetic: makes no HIP call.
 */
size_t slimkv_workspace_bytes(const slimkv_problem* problem, slimkv_op op);

/*
 * slimkv_decode_attn -- latent-space decode attention (the method itself).
 *
 *   q      [B, H_q, d]            decode query, before rotation
 *   q_pos  [B]          int32     absolute position of each decode query
 *   U_K    [H_kv, d, r_K]         beacon key basis of this layer
 *   U_V    [H_kv, d, r_V]         beacon value basis of this layer
 *   C_K    [B, H_kv, N_b, r_K]    latent beacon keys (no rotation)
 *   C_V    [B, H_kv, N_b, r_V]    latent beacon values
 *   K_raw  [B, H_kv, W, d]        raw keys, already rotated at their positions
 *   V_raw  [B, H_kv, W, d]        raw values
 *   out    [B, H_q, d]    fp32    attention output
 *   lse    [B, H_q]       fp32    log-sum-exp of the scaled scores, or NULL
 *
 * U_K, U_V, C_K, C_V may be NULL when N_b == 0; K_raw, V_raw may be NULL
 * when W == 0.
 */
slimkv_status slimkv_decode_attn(const slimkv_problem* problem, const void* q,
                                 const int32_t* q_pos, const void* U_K,
                                 const void* U_V, const void* C_K,
                                 const void* C_V, const void* K_raw,
                                 const void* V_raw, float* out, float* lse,
                                 void* workspace, size_t workspace_bytes,
                                 void* stream);

/*
 * slimkv_decode_attn_noalloc -- slimkv_decode_attn without a workspace
 * argument, for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.
 *
 * The workspace is a scratch array inside the library, one per device
 * (16 MiB, SLIMKV_NOALLOC_SCRATCH_BYTES, held until the process ends).  A
 * call needs 64 bytes per (b, kv head) unit plus (2 + d) * 4 bytes per query
 * head for each workgroup sharing a unit's rows (about 1.1 MB for batch 16,
 * 32/8 heads on a 256-CU device); a call that needs more than the scratch
 * holds returns SLIMKV_ERR_WORKSPACE and launches nothing (that check needs
 * the device's compute-unit count, a device query).  The call allocates and
 * frees nothing: it launches a small kernel that clears the scratch's
 * counters, then the attention kernel.  Every call on a device shares that
 * device's scratch and leaves its contents behind, so calls that can overlap
 * on one device (on different streams) race and must not be issued; calls
 * ordered on one stream are fine.  Results equal slimkv_decode_attn's with
 * the same problem (bitwise: same kernels, same split).  Arguments, layouts
 * and checks as for slimkv_decode_attn.
 */
#define SLIMKV_NOALLOC_SCRATCH_BYTES (16u << 20)

slimkv_status slimkv_decode_attn_noalloc(const slimkv_problem* problem, const void* q,
                                         const int32_t* q_pos, const void* U_K,
                                         const void* U_V, const void* C_K,
                                         const void* C_V, const void* K_raw,
                                         const void* V_raw, float* out, float* lse,
                                         void* stream);

/*
 * slimkv_decode_attn_ragged -- the same attention for one serving decode
 * step over a ragged batch, with the step's new token.
 *
 * Passages: page "Can SlimKV compress KV cache jointly across tokens and
 * features", section "Latent-space attention removes the rebuild step" (the
 * attention itself: raw-token keys keep rotation, beacon keys do not), and
 * section "Speedups are real, but memory is set by the ratio" (a decode run
 * generates tokens one at a time, so each step adds one raw-token row to the
 * cache it attends over); section "Why feature compression stalls at key
 * reconstruction" (the cache and its memory traffic are what limit
 * long-context serving, where sequences of a batch hold different lengths).
 * The pages do not spell out the cache update; the reading taken here is
 * append-then-attend: the new token is rotated at its own position, joins
 * the softmax as one more raw row, and is stored.
 *
 * The cache arrays are sized to capacities: problem->num_beacons is N_cap,
 * the beacon rows each (b, kv head) holds in C_K [B, H_kv, N_cap, r_K] and
 * C_V, and problem->raw_window is W_cap, the raw rows of K_raw, V_raw
 * [B, H_kv, W_cap, d].  Sequence b uses only its first
 *   n_b = clamp(num_beacons_b[b], 0, N_cap) beacon rows and
 *   w_b = clamp(raw_len[b], 0, W_cap) raw rows.
 * With k_new and v_new ([B, H_kv, d], the new token's key before rotation
 * and its value, in the problem dtype) the token joins sequence b as one
 * more raw row: its key is rotated at q_pos[b] (the decode token attends to
 * itself), computed in double precision and rounded once to the storage
 * dtype, and scored and summed like the other raw rows.  When w_b < W_cap
 * the call also stores that rotated key and the value as row w_b of
 * K_raw and V_raw (the only cache rows it writes; the caller then counts
 * the row in raw_len).  With a full window the token is attended but not
 * stored.  A sequence with no rows at all (no new token, n_b = w_b = 0)
 * gets out = 0 and lse = -inf.
 *
 *   num_beacons_b [B] int32  live beacon rows per sequence (device), or
 *                            NULL for N_cap each
 *   raw_len       [B] int32  live raw rows before this step (device), or
 *                            NULL for W_cap each
 *   k_new, v_new  [B, H_kv, d] the new token (device), both or neither
 *   K_raw, V_raw  written at the rows above when k_new is given
 * Other arguments as for slimkv_decode_attn.  N_cap + W_cap may be 0 (then
 * only the new token is attended).  The batch is at most 1024 sequences and
 * the only flag accepted is SLIMKV_FLAG_CHECK_WORKSPACE (the tiles of the
 * whole batch are shared out over the grid in a fixed order, so repeated
 * calls are bitwise equal).  Work is
 * shared out by tiles: each (b, kv head) gets workgroups in proportion to
 * its live rows, shaped for P workgroup slots -- the device's (num_splits
 * = 0) or num_splits -- with at most 64 per (b, kv head).  Workspace:
 * slimkv_workspace_bytes with SLIMKV_OP_LATENT_RAGGED, zero-filled before
 * first use, as for the other entry points.
 */
slimkv_status slimkv_decode_attn_ragged(const slimkv_problem* problem,
                                        const void* q, const int32_t* q_pos,
                                        const void* U_K, const void* U_V,
                                        const void* C_K, const void* C_V,
                                        void* K_raw, void* V_raw,
                                        const int32_t* num_beacons_b,
                                        const int32_t* raw_len,
                                        const void* k_new, const void* v_new,
                                        float* out, float* lse, void* workspace,
                                        size_t workspace_bytes, void* stream);

/*
 * Page tables of a paged cache (slimkv_decode_attn_paged).  Rows live in
 * fixed-size pages drawn from pools shared by the whole batch:
 *   C_K pool   [beacon_pages, H_kv, page_rows, r_K]
 *   C_V pool   [beacon_pages, H_kv, page_rows, r_V]
 *   K_raw pool [raw_pages,    H_kv, page_rows, d]
 *   V_raw pool [raw_pages,    H_kv, page_rows, d]
 * so one page holds page_rows consecutive rows of a sequence for all of its
 * KV heads.  Beacon row j of sequence b lies in page
 * beacon_table[b * beacon_table_width + j / page_rows] at row
 * j % page_rows; raw rows likewise through raw_table.  (40 bytes.)
 */
typedef struct slimkv_pages {
  int32_t page_rows;          /* rows per page: a power of two, 64 .. 65536     */
  int32_t beacon_pages;       /* pages in the C_K / C_V pools (>= 0)            */
  int32_t raw_pages;          /* pages in the K_raw / V_raw pools (>= 0)        */
  int32_t beacon_table_width; /* entries per sequence in beacon_table: at least
                                 ceil(N_cap / page_rows)                        */
  int32_t raw_table_width;    /* entries per sequence in raw_table: at least
                                 ceil(W_cap / page_rows)                        */
  int32_t reserved;           /* must be 0                                      */
  const int32_t* beacon_table; /* [B, beacon_table_width] int32 (device), or
                                  NULL when N_cap == 0                           */
  const int32_t* raw_table;    /* [B, raw_table_width] int32 (device), or NULL
                                  when W_cap == 0                                */
} slimkv_pages;

/*
 * slimkv_decode_attn_paged -- slimkv_decode_attn_ragged over a paged cache.
 *
 * Passages: as for slimkv_decode_attn_ragged.  The pages never mention
 * paging; it is read here as a storage indirection that changes no result,
 * so the defining computation stays the contiguous one.
 *
 * Computes exactly what slimkv_decode_attn_ragged computes for the logical
 * arrays the pages describe (out and lse are bitwise equal to that call's
 * on the same rows): the same clamped lengths n_b <= N_cap and w_b <= W_cap
 * (problem->num_beacons, problem->raw_window), the same new token, and the
 * same store of its rotated key and value as raw row w_b when w_b < W_cap,
 * here into the page that raw_table gives for that row.  The call reads
 * only the table entries of pages that hold live rows (and of the page
 * that receives the new token), and only the live rows of those pages.
 * A table entry outside [0, pages) reads as a page of zeros and is never
 * written; the library never touches memory outside the pools.  Pages may
 * be shared between sequences (a common prefix) except for a page that
 * receives a new token in this call.  ceil(N_cap / page_rows) +
 * ceil(W_cap / page_rows) must not exceed 4096 (the tables of a sequence are
 * staged on chip).
 *
 *   pages              host struct above; its tables are device memory
 *   C_K, C_V           beacon pools (NULL when N_cap == 0)
 *   K_raw, V_raw       raw pools (NULL when W_cap == 0); written only at the
 *                      new token's rows
 * Other arguments, limits and the workspace (slimkv_workspace_bytes with
 * SLIMKV_OP_LATENT_RAGGED) as for slimkv_decode_attn_ragged.
 */
slimkv_status slimkv_decode_attn_paged(const slimkv_problem* problem,
                                       const slimkv_pages* pages,
                                       const void* q, const int32_t* q_pos,
                                       const void* U_K, const void* U_V,
                                       const void* C_K, const void* C_V,
                                       void* K_raw, void* V_raw,
                                       const int32_t* num_beacons_b,
                                       const int32_t* raw_len,
                                       const void* k_new, const void* v_new,
                                       float* out, float* lse, void* workspace,
                                       size_t workspace_bytes, void* stream);

/*
 * slimkv_decode_attn_chunk -- the same attention for a chunk of Q query
 * tokens per sequence: speculative decoding checks several drafted tokens
 * in one pass, chunked prefill feeds a prompt Q tokens at a time.
 *
 * Passages: page "Can SlimKV compress KV cache jointly across tokens and
 * features", section "Latent-space attention removes the rebuild step" (the
 * attention for every query: rotated, grouped, projected into the beacon
 * latent space), and section "Speedups are real, but memory is set by the
 * ratio" (time-to-first-token, i.e. queries that arrive several at a time,
 * gains from skipping full-key materialisation too).  With Q queries per
 * KV head the latent products become dense, so they run on the matrix
 * cores.  Causality among the chunk's own tokens is the ordinary decoder
 * reading: token t sees tokens 0 .. t.
 *
 * Token t
 * of sequence b sits at position q_pos[b] + t.  Each of its query heads is
 * rotated there and attends, under one softmax, over the sequence's live
 * beacon rows (latent, as in slimkv_decode_attn), its live raw rows, and the
 * chunk's new tokens 0 .. t -- token u's key rotated at q_pos[b] + u in
 * double precision and rounded once to the cache dtype -- but not over the chunk's
 * later tokens.  The tokens u with w_b + u < W_cap are then stored as raw
 * rows w_b + u of K_raw and V_raw (rotated key, value); the others are
 * attended but not stored.  Without k_new and v_new every query of the
 * chunk attends over the cache rows only.  With Q = 1 this is
 * slimkv_decode_attn_ragged.
 *
 *   num_tokens    Q >= 1, with (H_q / H_kv) * Q <= 16 (the query rows of one
 *                 KV head fill one matrix-core tile)
 *   q             [B, Q, H_q, d]   the chunk's queries, before rotation
 *   k_new, v_new  [B, Q, H_kv, d]  the chunk's tokens (key before rotation),
 *                                  both or neither
 *   out           [B, Q, H_q, d] fp32;  lse [B, Q, H_q] fp32 or NULL
 * Capacity-sized caches, lengths, clamping, limits (batch <= 1024, flags as
 * for the ragged call)
 * and num_splits as for slimkv_decode_attn_ragged.  bf16 or fp32 caches
 * (fp32: the products on the fp32 matrix instructions).  Workspace:
 * slimkv_chunk_workspace_bytes(problem, num_tokens) bytes, zero-filled
 * before first use.
 */
size_t slimkv_chunk_workspace_bytes(const slimkv_problem* problem, int32_t num_tokens);

slimkv_status slimkv_decode_attn_chunk(const slimkv_problem* problem,
                                       int32_t num_tokens, const void* q,
                                       const int32_t* q_pos, const void* U_K,
                                       const void* U_V, const void* C_K,
                                       const void* C_V, void* K_raw, void* V_raw,
                                       const int32_t* num_beacons_b,
                                       const int32_t* raw_len,
                                       const void* k_new, const void* v_new,
                                       float* out, float* lse, void* workspace,
                                       size_t workspace_bytes, void* stream);

/*
 * slimkv_decode_attn_chunk_paged -- slimkv_decode_attn_chunk over a paged
 * cache (speculative decoding in a serving engine whose cache lives in
 * pages).
 *
 * Passages: as for slimkv_decode_attn_chunk; paging as for
 * slimkv_decode_attn_paged (a storage indirection that changes no result).
 *
 * Computes exactly what slimkv_decode_attn_chunk computes for the logical
 * arrays the pages describe (out and lse are bitwise equal to that call's
 * on the same rows), with the pools, tables and their rules as for
 * slimkv_decode_attn_paged: the chunk's tokens u with w_b + u < W_cap are
 * stored as raw rows w_b + u in the pages raw_table gives for those rows
 * (not where an entry is outside [0, raw_pages)), and a page that receives
 * a token in this call must not be shared.  The call reads the table
 * entries of pages that hold live rows or receive tokens.
 *
 *   pages         host struct as for slimkv_decode_attn_paged
 *   C_K, C_V      beacon pools (NULL when N_cap == 0)
 *   K_raw, V_raw  raw pools (NULL when W_cap == 0); written only at the
 *                 chunk's tokens' rows
 * Other arguments, limits and the workspace (slimkv_chunk_workspace_bytes)
 * as for slimkv_decode_attn_chunk.
 */
slimkv_status slimkv_decode_attn_chunk_paged(const slimkv_problem* problem,
                                             const slimkv_pages* pages,
                                             int32_t num_tokens, const void* q,
                                             const int32_t* q_pos, const void* U_K,
                                             const void* U_V, const void* C_K,
                                             const void* C_V, void* K_raw, void* V_raw,
                                             const int32_t* num_beacons_b,
                                             const int32_t* raw_len,
                                             const void* k_new, const void* v_new,
                                             float* out, float* lse, void* workspace,
                                             size_t workspace_bytes, void* stream);

/*
 * slimkv_decode_attn_alibi -- the latent decode attention of an ALiBi
 * backbone.  Page "Can SlimKV compress KV cache jointly across tokens and
 * features" notes that ALiBi adds its positional bias after the query-key
 * product, so it composes with the latent beacon scores.  Such a backbone
 * has no rotary embedding: neither the query nor any key is rotated (raw
 * keys are stored as they are), and each score gets
 *   s_j = scale * (q . k_j) - slopes[h_q] * (q_pos[b] - pos_j)
 * (beacon scores in latent form, (q U_K) . C_K[j], as in
 * slimkv_decode_attn), with the query head's slope, before the softmax.
 * Key positions:
 *   beacon j   pos_j = beacon_first + j * beacon_stride (e.g. one beacon
 *              per s tokens at its last token: first s - 1, stride s);
 *   raw row t  pos = q_pos[b] - W + 1 + t (the window ends at the query).
 *
 *   slopes  [H_q] fp32 (device), e.g. the ALiBi paper's geometric slopes
 * beacon_first >= 0, beacon_stride >= 0 and the last beacon's position
 * must fit in int32; distances are formed in int32 and converted to fp32
 * (exact below 2^24).  Other arguments, layouts and the workspace
 * (slimkv_workspace_bytes with SLIMKV_OP_LATENT) as for slimkv_decode_attn;
 * rope_theta is unused but still checked.
 */
slimkv_status slimkv_decode_attn_alibi(const slimkv_problem* problem,
                                       const void* q, const int32_t* q_pos,
                                       const void* U_K, const void* U_V,
                                       const void* C_K, const void* C_V,
                                       const void* K_raw, const void* V_raw,
                                       const float* slopes, int32_t beacon_first,
                                       int32_t beacon_stride, float* out, float* lse,
                                       void* workspace, size_t workspace_bytes,
                                       void* stream);

/*
 * ALiBi forms of the serving calls.  The same steps as
 * slimkv_decode_attn_ragged, _paged, _chunk and _chunk_paged, for an ALiBi
 * backbone (page "Can SlimKV compress KV cache jointly across tokens and
 * features", section "Latent-space attention removes the rebuild step":
 * ALiBi adds its positional bias after the query-key product, so it
 * composes with the latent beacon scores).  As in slimkv_decode_attn_alibi
 * nothing is rotated -- not the queries, not the raw keys, not the new
 * tokens, which are scored and stored as given -- and every score gets
 *   -slopes[h_q] * (q_pos_t - k_pos)
 * after the scaled product.  Positions, for sequence b with w_b live raw
 * rows (the reading of a window that ends at the newest token):
 *   query token t       q_pos[b] + t
 *   beacon j            beacon_first + j * beacon_stride
 *   new token u         q_pos[b] + u
 *   live raw row i      q_pos[b] - w_b + i when the call brings new tokens
 *                       (they follow the raw rows); q_pos[b] - w_b + 1 + i
 *                       without (the first query's own token is the last
 *                       raw row, as in slimkv_decode_attn_alibi)
 * Distances are formed in int32 and converted to fp32 (exact below 2^24).
 * Every other argument, limit and rule (lengths, clamping, the stores of
 * new tokens, pages, workspace) is that of the rotary call of the same name
 * without _alibi; problem->rope_theta is unused but still checked.
 */
typedef struct slimkv_alibi {
  const float* slopes;    /* [H_q] fp32 (device), e.g. the ALiBi paper's slopes */
  int32_t beacon_first;   /* position of beacon 0, >= 0                        */
  int32_t beacon_stride;  /* positions between consecutive beacons, >= 0;
                             the last beacon's position must fit in int32      */
} slimkv_alibi;

slimkv_status slimkv_decode_attn_ragged_alibi(const slimkv_problem* problem,
                                              const slimkv_alibi* alibi, const void* q,
                                              const int32_t* q_pos, const void* U_K,
                                              const void* U_V, const void* C_K, const void* C_V,
                                              void* K_raw, void* V_raw,
                                              const int32_t* num_beacons_b, const int32_t* raw_len,
                                              const void* k_new, const void* v_new, float* out,
                                              float* lse, void* workspace, size_t workspace_bytes,
                                              void* stream);
slimkv_status slimkv_decode_attn_paged_alibi(const slimkv_problem* problem,
                                             const slimkv_pages* pages, const slimkv_alibi* alibi,
                                             const void* q, const int32_t* q_pos, const void* U_K,
                                             const void* U_V, const void* C_K, const void* C_V,
                                             void* K_raw, void* V_raw,
                                             const int32_t* num_beacons_b, const int32_t* raw_len,
                                             const void* k_new, const void* v_new, float* out,
                                             float* lse, void* workspace, size_t workspace_bytes,
                                             void* stream);
slimkv_status slimkv_decode_attn_chunk_alibi(const slimkv_problem* problem,
                                             const slimkv_alibi* alibi, int32_t num_tokens,
                                             const void* q, const int32_t* q_pos, const void* U_K,
                                             const void* U_V, const void* C_K, const void* C_V,
                                             void* K_raw, void* V_raw,
                                             const int32_t* num_beacons_b, const int32_t* raw_len,
                                             const void* k_new, const void* v_new, float* out,
                                             float* lse, void* workspace, size_t workspace_bytes,
                                             void* stream);
slimkv_status slimkv_decode_attn_chunk_paged_alibi(
    const slimkv_problem* problem, const slimkv_pages* pages, const slimkv_alibi* alibi,
    int32_t num_tokens, const void* q, const int32_t* q_pos, const void* U_K, const void* U_V,
    const void* C_K, const void* C_V, void* K_raw, void* V_raw, const int32_t* num_beacons_b,
    const int32_t* raw_len, const void* k_new, const void* v_new, float* out, float* lse,
    void* workspace, size_t workspace_bytes, void* stream);

/*
 * slimkv_reconstruct_attn -- comparison path: the decode step of the
 * reconstruction-based variant timed against SlimKV on the same page
 * (section "Speedups are real, but memory is set by the ratio"): beacon keys
 * and values are first rebuilt at full dimension, K_b = C_K U_K^T and
 * V_b = C_V U_V^T, written to the workspace in the problem dtype, and then
 * attended together with the raw rows by ordinary attention.  The rebuilt
 * beacon keys get no rotation here, so in exact arithmetic the result
 * equals slimkv_decode_attn's; it differs only by the rounding of K_b, V_b
 * to the storage dtype.  Same arguments and layouts as slimkv_decode_attn.
 */
slimkv_status slimkv_reconstruct_attn(const slimkv_problem* problem,
                                      const void* q, const int32_t* q_pos,
                                      const void* U_K, const void* U_V,
                                      const void* C_K, const void* C_V,
                                      const void* K_raw, const void* V_raw,
                                      float* out, float* lse, void* workspace,
                                      size_t workspace_bytes, void* stream);

/*
 * slimkv_reconstruct_rope_attn -- the reconstruction variant exactly as the
 * same section times it: it keeps the rotation of beacon keys.  Beacon keys
 * and values are rebuilt at full dimension into the workspace as in
 * slimkv_reconstruct_attn, but each rebuilt key K_b[j] = U_K C_K[j] is
 * rotated at position beacon_pos[j] (rotate-half pairs, angle
 * beacon_pos[j] * theta^(-2i/d)) before it is rounded to the dtype; the
 * rotated query then attends over the rebuilt and raw rows.  This is not
 * the latent result (SlimKV's beacon keys carry no rotation); it is the
 * baseline the SlimKV timings are compared with.
 *
 *   beacon_pos [N_b] int32 (device)  position of beacon j, the same for
 *                                     every sequence (e.g. (j + 1) * s - 1
 *                                     for one beacon per s tokens); may be
 *                                     NULL when N_b == 0
 * Other arguments, layouts and the workspace (slimkv_workspace_bytes with
 * SLIMKV_OP_RECONSTRUCT) as for slimkv_reconstruct_attn.
 */
slimkv_status slimkv_reconstruct_rope_attn(const slimkv_problem* problem,
                                           const void* q, const int32_t* q_pos,
                                           const void* U_K, const void* U_V,
                                           const void* C_K, const void* C_V,
                                           const void* K_raw, const void* V_raw,
                                           const int32_t* beacon_pos, float* out,
                                           float* lse, void* workspace,
                                           size_t workspace_bytes, void* stream);

/*
 * full_kv_attn -- comparison path: uncompressed grouped-query decode
 * attention over all T cached tokens (the "Full KV" baseline of the same
 * section).  The problem must have num_beacons == 0 and raw_window == T.
 *
 *   q [B, H_q, d], q_pos [B] int32 as above;
 *   K [B, H_kv, T, d] keys already rotated at their positions; V [B, H_kv, T, d];
 *   out [B, H_q, d] fp32; lse [B, H_q] fp32 or NULL.
 */
slimkv_status full_kv_attn(const slimkv_problem* problem, const void* q,
                           const int32_t* q_pos, const void* K, const void* V,
                           float* out, float* lse, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * Profiling hook (optional).  The next successful entry-point call made on
 * this thread records `start` right before it launches its attention kernel
 * (the kernel that streams the cache) and `stop` right after, both on the
 * call's stream, then forgets them.  start and stop are hipEvent_t handles
 * owned by the caller; NULL, NULL clears a pending pair.  Lets a caller time
 * that one kernel with events; the computation is unchanged.
 */
slimkv_status slimkv_set_kernel_events(void* start, void* stop);

/* Static text for a status code. */
const char* slimkv_status_string(slimkv_status status);

/* Detail of the last failed call on this thread ("" if none). */
const char* slimkv_last_error(void);

/*
 * The status word of a workspace (4 bytes at its start): 0 while every call
 * made with SLIMKV_FLAG_CHECK_WORKSPACE found the counters and flags at
 * zero; bit 0 set once one did not.  Zero-filling the workspace clears it.
 * Debugging aid: copies the word to the host with a synchronous hipMemcpy,
 * so it waits for the device.
 */
slimkv_status slimkv_workspace_status(const void* workspace, uint32_t* status);

/* SLIMKV_ABI_VERSION of the loaded library. */
int32_t slimkv_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SLIMKV_H */
