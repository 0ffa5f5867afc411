// api.cpp -- the C ABI declared in include/slimkv.h: argument checks, the
// split plan, workspace layout and the launch sequence of each entry point.
//
// Every check runs before the first HIP call, so a rejected call launches
// nothing, touches no output and works on a machine without a GPU.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <string>

#include "internal.h"
#include "slimkv.h"

static_assert(slimkv::kNoAllocScratchBytes == SLIMKV_NOALLOC_SCRATCH_BYTES,
              "the header states the scratch size");

namespace slimkv {
namespace {

thread_local std::string g_last_error;
thread_local hipEvent_t g_ev_start = nullptr, g_ev_stop = nullptr;

slimkv_status fail(slimkv_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

// rows per unit and segment: a unit's rows are addressed with 32-bit byte
// offsets (at most 2^22 rows x 512 bytes)
constexpr int64_t kMaxRows = int64_t(1) << 22;
constexpr int64_t kMaxUnits = int64_t(1) << 20;   // batch * kv heads
constexpr size_t kAlign = 256;                    // workspace sub-buffer alignment

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct Plan {
  AttnArgs attn;
  int64_t units;
  int dtype;
  int elem;
  size_t off_counters, off_flags, off_ml, off_acc, off_kb, off_vb, total;
};

bool rank_ok(int r) { return r >= 16 && r <= kHeadDim && r % 16 == 0; }

// Shape checks shared by every op.  For full_kv_attn num_beacons must be 0.
slimkv_status check_problem(const slimkv_problem* p, slimkv_op op) {
  if (!p) return fail(SLIMKV_ERR_NULL, "problem is NULL");
  if (op != SLIMKV_OP_LATENT && op != SLIMKV_OP_RECONSTRUCT && op != SLIMKV_OP_FULL_KV &&
      op != SLIMKV_OP_LATENT_RAGGED)
    return fail(SLIMKV_ERR_UNSUPPORTED, "unknown op %d", (int)op);
  const bool ragged = op == SLIMKV_OP_LATENT_RAGGED;
  if ((p->flags & ~(SLIMKV_FLAG_DYNAMIC_TILES | SLIMKV_FLAG_CHECK_WORKSPACE)) != 0)
    return fail(SLIMKV_ERR_SHAPE, "unknown flag bits 0x%x", (unsigned)p->flags);
  if (ragged && (p->flags & SLIMKV_FLAG_DYNAMIC_TILES) != 0)
    return fail(SLIMKV_ERR_UNSUPPORTED, "ragged calls deal their tiles in a fixed order only");
  if (ragged && p->batch > kMaxRaggedBatch)
    return fail(SLIMKV_ERR_UNSUPPORTED, "ragged batch %d exceeds %d", p->batch, kMaxRaggedBatch);
  if (p->dtype != SLIMKV_FP32 && p->dtype != SLIMKV_BF16)
    return fail(SLIMKV_ERR_UNSUPPORTED, "dtype %d is not fp32 (0) or bf16 (1)", p->dtype);
  if (p->batch < 1 || p->num_q_heads < 1 || p->num_kv_heads < 1)
    return fail(SLIMKV_ERR_SHAPE, "batch, num_q_heads and num_kv_heads must be >= 1");
  if (p->num_q_heads % p->num_kv_heads != 0)
    return fail(SLIMKV_ERR_SHAPE, "num_q_heads %d is not a multiple of num_kv_heads %d",
                p->num_q_heads, p->num_kv_heads);
  if (p->num_q_heads / p->num_kv_heads > kMaxGroup)
    return fail(SLIMKV_ERR_UNSUPPORTED, "group size %d exceeds %d",
                p->num_q_heads / p->num_kv_heads, kMaxGroup);
  if ((int64_t)p->batch * p->num_kv_heads > kMaxUnits)
    return fail(SLIMKV_ERR_UNSUPPORTED, "batch * num_kv_heads exceeds %lld", (long long)kMaxUnits);
  if (p->head_dim != kHeadDim)
    return fail(SLIMKV_ERR_UNSUPPORTED, "head_dim %d is not %d", p->head_dim, kHeadDim);
  if (p->num_beacons < 0 || p->raw_window < 0)
    return fail(SLIMKV_ERR_SHAPE, "num_beacons and raw_window must be >= 0");
  if (!ragged && (int64_t)p->num_beacons + p->raw_window < 1)
    return fail(SLIMKV_ERR_SHAPE, "num_beacons + raw_window must be >= 1");
  if (p->num_beacons > kMaxRows || p->raw_window > kMaxRows)
    return fail(SLIMKV_ERR_UNSUPPORTED, "more than %lld rows per unit", (long long)kMaxRows);
  if (op == SLIMKV_OP_FULL_KV && p->num_beacons != 0)
    return fail(SLIMKV_ERR_SHAPE, "full_kv_attn needs num_beacons == 0 (raw_window is T)");
  if (p->num_beacons > 0 && (!rank_ok(p->rank_k) || !rank_ok(p->rank_v)))
    return fail(SLIMKV_ERR_UNSUPPORTED,
                "rank_k %d / rank_v %d: each must be a multiple of 16 in [16, %d]", p->rank_k,
                p->rank_v, kHeadDim);
  if (!(p->scale > 0.0f) || !isfinite(p->scale))
    return fail(SLIMKV_ERR_SHAPE, "scale must be finite and > 0");
  if (!(p->rope_theta > 1.0) || !isfinite(p->rope_theta))
    return fail(SLIMKV_ERR_SHAPE, "rope_theta must be finite and > 1");
  if (p->num_splits < 0) return fail(SLIMKV_ERR_SHAPE, "num_splits must be >= 0");
  return SLIMKV_OK;
}

slimkv_status make_plan(const slimkv_problem* p, slimkv_op op, Plan& pl) {
  slimkv_status st = check_problem(p, op);
  if (st != SLIMKV_OK) return st;
  memset(&pl, 0, sizeof pl);
  pl.dtype = p->dtype;
  pl.elem = p->dtype == SLIMKV_FP32 ? 4 : 2;
  pl.units = (int64_t)p->batch * p->num_kv_heads;
  AttnArgs& a = pl.attn;
  a.batch = p->batch;
  a.num_q_heads = p->num_q_heads;
  a.num_kv_heads = p->num_kv_heads;
  a.group = p->num_q_heads / p->num_kv_heads;

  // seg[0]: beacon rows (latent, or rebuilt at full width); seg[1]: raw rows.
  // An absent segment has rows = 0.
  Segment& sb = a.seg[0];
  sb.rows = p->num_beacons;
  if ((op == SLIMKV_OP_LATENT || op == SLIMKV_OP_LATENT_RAGGED) && p->num_beacons > 0) {
    sb.kind = kSegLatent;
    sb.rk = p->rank_k;
    sb.rv = p->rank_v;
  } else {
    sb.kind = kSegFull;
    sb.rk = sb.rv = kHeadDim;
  }
  Segment& sr = a.seg[1];
  sr.kind = kSegFull;
  sr.rows = p->raw_window;
  sr.rk = sr.rv = kHeadDim;
  for (Segment* sg : {&sb, &sr}) {
    sg->row_bytes = (sg->rk + sg->rv) * pl.elem;
    sg->tile = tile_rows(pl.dtype, sg->rk, sg->rv);
  }
  a.unit_bytes = (int64_t)sb.rows * sb.row_bytes + (int64_t)sr.rows * sr.row_bytes;
  // 0: the launcher picks; ragged calls read num_splits as the workgroup
  // slots the pieces are shaped for (the launcher caps it), the others as
  // workgroups per unit
  a.chunks = p->num_splits <= 0 ? 0
             : (op == SLIMKV_OP_LATENT_RAGGED ? p->num_splits : std::min(p->num_splits, kMaxChunks));
  a.deterministic = (p->flags & SLIMKV_FLAG_DYNAMIC_TILES) == 0;
  if (pl.units * kMaxChunks > (int64_t)INT32_MAX)
    return fail(SLIMKV_ERR_UNSUPPORTED, "too many workgroups");
  const bool ragged = op == SLIMKV_OP_LATENT_RAGGED;
  if (ragged) {
    // tile positions of the whole batch are 32-bit
    const int64_t tiles = ceil_div(sb.rows, sb.tile) + ceil_div(sr.rows, sr.tile);
    if (pl.units * tiles > (int64_t)INT32_MAX)
      return fail(SLIMKV_ERR_UNSUPPORTED, "too many tiles in the batch");
  }
  a.rank_v = sb.kind == kSegLatent ? p->rank_v : 0;
  a.rank_k = sb.kind == kSegLatent ? p->rank_k : 0;

  // workspace layout: per-unit counters and per-slot flags (must start
  // zeroed), then one partial slot per workgroup for up to kMaxChunks
  // workgroups per unit (ragged: one per piece, fewer than grid + units)
  const int64_t G = a.group, slots = ragged ? kMaxChunks + 1 : kMaxChunks;
  pl.off_counters = kWsHeader;
  size_t off = round_up(kWsHeader + pl.units * kCounterStride * sizeof(uint32_t), kAlign);
  pl.off_flags = off;
  off = round_up(off + (size_t)(pl.units * slots) * sizeof(uint32_t), kAlign);
  pl.off_ml = off;
  off = round_up(off + (size_t)(pl.units * slots * G * 2) * sizeof(float), kAlign);
  pl.off_acc = off;
  off = round_up(off + (size_t)(pl.units * slots * G * kHeadDim) * sizeof(float), kAlign);
  pl.off_kb = pl.off_vb = off;
  if (op == SLIMKV_OP_RECONSTRUCT && p->num_beacons > 0) {
    const size_t rebuilt = (size_t)pl.units * p->num_beacons * kHeadDim * pl.elem;
    off = round_up(off + rebuilt, kAlign);
    pl.off_vb = off;
    off = round_up(off + rebuilt, kAlign);
  }
  pl.total = off;
  return SLIMKV_OK;
}

// Plan of a chunk call: the ragged call's segments and schedule limits,
// G * Q <= kChunkRows query rows per unit; partial slots for
// every piece the launcher can make (at most units + kChunkMaxSlots), each
// holding G * Q rows.
slimkv_status make_chunk_plan(const slimkv_problem* p, int32_t num_tokens, Plan& pl) {
  slimkv_status st = make_plan(p, SLIMKV_OP_LATENT_RAGGED, pl);
  if (st != SLIMKV_OK) return st;
  const int G = p->num_q_heads / p->num_kv_heads;
  if (num_tokens < 1) return fail(SLIMKV_ERR_SHAPE, "num_tokens must be >= 1");
  if ((int64_t)G * num_tokens > kChunkRows)
    return fail(SLIMKV_ERR_UNSUPPORTED, "group %d x %d tokens exceeds %d query rows per KV head", G,
                num_tokens, kChunkRows);
  // slots: the pieces' (at most max(units, kChunkMaxSlots)), then one for
  // each unit's tokens
  const int64_t M = (int64_t)G * num_tokens, slots = 2 * pl.units + kChunkMaxSlots;
  pl.attn.num_tokens = num_tokens;
  pl.off_counters = kWsHeader;
  size_t off = round_up(kWsHeader + pl.units * kCounterStride * sizeof(uint32_t), kAlign);
  pl.off_flags = off;
  off = round_up(off + (size_t)slots * sizeof(uint32_t), kAlign);
  pl.off_ml = off;
  off = round_up(off + (size_t)(slots * M * 2) * sizeof(float), kAlign);
  pl.off_acc = off;
  off = round_up(off + (size_t)(slots * M * kHeadDim) * sizeof(float), kAlign);
  pl.off_kb = pl.off_vb = off;
  pl.total = off;
  return SLIMKV_OK;
}

struct Range {
  const void* p;
  size_t bytes;
  const char* name;
};

bool overlap(const Range& x, const Range& y) {
  if (!x.p || !y.p || !x.bytes || !y.bytes) return false;
  const uintptr_t a0 = (uintptr_t)x.p, a1 = a0 + x.bytes;
  const uintptr_t b0 = (uintptr_t)y.p, b1 = b0 + y.bytes;
  return a0 < b1 && b0 < a1;
}

// Pointer checks: presence, alignment, and outputs not overlapping inputs
// or each other.
slimkv_status check_pointers(const Range* in, int n_in, const Range* req, int n_req,
                             const Range* outs, int n_out, int align_req) {
  for (int i = 0; i < n_req; ++i)
    if (!req[i].p) return fail(SLIMKV_ERR_NULL, "%s is NULL", req[i].name);
  for (int i = 0; i < n_in; ++i)
    if (in[i].p && ((uintptr_t)in[i].p % (in[i].bytes == 0 ? 1 : (uintptr_t)align_req)) != 0)
      return fail(SLIMKV_ERR_ALIGN, "%s is not %d-byte aligned", in[i].name, align_req);
  for (int i = 0; i < n_out; ++i) {
    if (outs[i].p && (uintptr_t)outs[i].p % 4 != 0)
      return fail(SLIMKV_ERR_ALIGN, "%s is not 4-byte aligned", outs[i].name);
    for (int j = 0; j < n_in; ++j)
      if (overlap(outs[i], in[j]))
        return fail(SLIMKV_ERR_ALIAS, "%s overlaps %s", outs[i].name, in[j].name);
    for (int j = 0; j < i; ++j)
      if (overlap(outs[i], outs[j]))
        return fail(SLIMKV_ERR_ALIAS, "%s overlaps %s", outs[i].name, outs[j].name);
  }
  return SLIMKV_OK;
}

// ALiBi parameters of a latent call (slopes null: a rotary call)
struct Alibi {
  const float* slopes = nullptr;  // [H_q] (device)
  int32_t first = 0, stride = 0;  // beacon j at first + j * stride
};

// Checks of an ALiBi call's parameters (slopes set): positions of the
// beacons fit in int32, the slopes are 4-byte aligned.
slimkv_status check_alibi(const slimkv_problem* p, const Alibi& alibi) {
  if (!alibi.slopes) return SLIMKV_OK;
  const int64_t last = (int64_t)alibi.first + (int64_t)std::max(p->num_beacons - 1, 0) * alibi.stride;
  if (alibi.stride < 0 || alibi.first < 0 || last > INT32_MAX)
    return fail(SLIMKV_ERR_SHAPE, "beacon positions first %d + j * stride %d must be >= 0 and "
                "fit in int32", alibi.first, alibi.stride);
  if ((uintptr_t)alibi.slopes % 4 != 0) return fail(SLIMKV_ERR_ALIGN, "slopes is not 4-byte aligned");
  return SLIMKV_OK;
}

// noalloc: the workspace is the library's device scratch (ws must be NULL;
// slimkv_decode_attn_noalloc), laid out for the chunk count this call uses.
slimkv_status run(const slimkv_problem* p, slimkv_op op, const void* q, const int32_t* q_pos,
                  const void* U_K, const void* U_V, const void* C_K, const void* C_V,
                  const void* K_raw, const void* V_raw, float* out, float* lse, void* ws,
                  size_t ws_bytes, void* stream, const int32_t* beacon_pos = nullptr,
                  const Alibi& alibi = Alibi(), bool noalloc = false) {
  Plan pl;
  slimkv_status st = make_plan(p, op, pl);
  if (st != SLIMKV_OK) return st;
  st = check_alibi(p, alibi);
  if (st != SLIMKV_OK) return st;
  const size_t e = (size_t)pl.elem;
  const size_t B = p->batch, Hq = p->num_q_heads, Hkv = p->num_kv_heads, d = kHeadDim;
  const size_t nb = p->num_beacons, w = p->raw_window;
  const bool beacons = nb > 0, raw = w > 0;
  const size_t rk = beacons ? p->rank_k : 0, rv = beacons ? p->rank_v : 0;

  Range in[8] = {
      {q, B * Hq * d * e, "q"},
      {q_pos, B * sizeof(int32_t), "q_pos"},
      {beacons ? U_K : nullptr, Hkv * d * rk * e, "U_K"},
      {beacons ? U_V : nullptr, Hkv * d * rv * e, "U_V"},
      {beacons ? C_K : nullptr, B * Hkv * nb * rk * e, "C_K"},
      {beacons ? C_V : nullptr, B * Hkv * nb * rv * e, "C_V"},
      {raw ? K_raw : nullptr, B * Hkv * w * d * e, op == SLIMKV_OP_FULL_KV ? "K" : "K_raw"},
      {raw ? V_raw : nullptr, B * Hkv * w * d * e, op == SLIMKV_OP_FULL_KV ? "V" : "V_raw"},
  };
  Range req[9];
  int n_req = 0;
  req[n_req++] = in[0];
  req[n_req++] = in[1];
  if (beacons)
    for (int i = 2; i < 6; ++i) req[n_req++] = in[i];
  if (raw) {
    req[n_req++] = in[6];
    req[n_req++] = in[7];
  }
  req[n_req++] = Range{out, 1, "out"};
  Range outs[3] = {{out, B * Hq * d * sizeof(float), "out"},
                   {lse, lse ? B * Hq * sizeof(float) : 0, "lse"},
                   {ws, pl.total, "workspace"}};
  // q_pos only needs int32 alignment; everything read as 16-byte vectors needs 16
  Range in16[8];
  int n16 = 0;
  for (int i = 0; i < 8; ++i)
    if (i != 1) in16[n16++] = in[i];
  if ((uintptr_t)q_pos % 4 != 0) return fail(SLIMKV_ERR_ALIGN, "q_pos is not 4-byte aligned");
  st = check_pointers(in16, n16, req, n_req, outs, 3, 16);
  if (st != SLIMKV_OK) return st;
  if (overlap(outs[0], in[1]) || overlap(outs[1], in[1]) || overlap(outs[2], in[1]))
    return fail(SLIMKV_ERR_ALIAS, "an output overlaps q_pos");
  if (alibi.slopes) {
    const Range sl{alibi.slopes, Hq * sizeof(float), "slopes"};
    for (const Range& o : outs)
      if (overlap(o, sl)) return fail(SLIMKV_ERR_ALIAS, "%s overlaps slopes", o.name);
  }
  if (beacon_pos) {
    const Range bp{beacon_pos, nb * sizeof(int32_t), "beacon_pos"};
    if ((uintptr_t)beacon_pos % 4 != 0) return fail(SLIMKV_ERR_ALIGN, "beacon_pos is not 4-byte aligned");
    for (const Range& o : outs)
      if (overlap(o, bp)) return fail(SLIMKV_ERR_ALIAS, "%s overlaps beacon_pos", o.name);
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  AttnArgs& a = pl.attn;
  if (!noalloc) {
    if (!ws) return fail(SLIMKV_ERR_NULL, "workspace is NULL");
    if ((uintptr_t)ws % 16 != 0) return fail(SLIMKV_ERR_ALIGN, "workspace is not 16-byte aligned");
    if (ws_bytes < pl.total)
      return fail(SLIMKV_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, pl.total);
  } else {
    // The scratch holds the counters and one partial slot per workgroup of
    // this call: the chunk count is fixed here (as the launcher would pick
    // it), which needs the device's workgroup slots -- a device query; no
    // launch happens before every check has passed.
    if (a.chunks <= 0) {
      const int slots = attention_slots(a, pl.dtype);
      if (slots <= 0) return fail(SLIMKV_ERR_HIP, "device query failed");
      a.chunks = choose_chunks(pl.units, a.unit_bytes, slots, 64 << 10);
    }
    const size_t G = a.group, k = a.chunks;
    pl.off_counters = kWsHeader;
    size_t off = round_up(kWsHeader + pl.units * kCounterStride * sizeof(uint32_t), kAlign);
    pl.off_flags = off;
    off = round_up(off + pl.units * k * sizeof(uint32_t), kAlign);
    pl.off_ml = off;
    off = round_up(off + pl.units * k * G * 2 * sizeof(float), kAlign);
    pl.off_acc = off;
    pl.total = round_up(off + pl.units * k * G * kHeadDim * sizeof(float), kAlign);
    if (pl.total > kNoAllocScratchBytes)
      return fail(SLIMKV_ERR_WORKSPACE,
                  "this call needs %zu bytes of scratch (%lld units x %zu workgroups); the "
                  "no-alloc entry point holds %zu (use slimkv_decode_attn with a workspace)",
                  pl.total, (long long)pl.units, k, kNoAllocScratchBytes);
    const hipError_t e = noalloc_scratch(pl.off_ml, s, &ws);
    if (e != hipSuccess) return fail(SLIMKV_ERR_HIP, "scratch set-up failed: %s", hipGetErrorString(e));
  }

  // ---- all checks passed: launch
  char* wsb = static_cast<char*>(ws);
  a.q = q;
  a.q_pos = q_pos;
  a.U_K = U_K;
  a.U_V = U_V;
  for (int k = 0; k < 6; ++k)  // rotary frequencies theta^(-2i/d), i < d/2 = 64
    a.inv_freq_pow2[k] = pow(p->rope_theta, -2.0 * (double)(1 << k) / (double)kHeadDim);
  a.score_scale = (double)p->scale * 1.4426950408889634074;  // scale * log2(e)
  a.counters = reinterpret_cast<uint32_t*>(wsb + pl.off_counters);
  a.flags = reinterpret_cast<uint32_t*>(wsb + pl.off_flags);
  a.part_ml = reinterpret_cast<float*>(wsb + pl.off_ml);
  a.part_acc = reinterpret_cast<float*>(wsb + pl.off_acc);
  a.out = out;
  a.lse = lse;
  a.alibi_slopes = alibi.slopes;
  a.beacon_first = alibi.first;
  a.beacon_stride = alibi.stride;
  if (beacons) {
    a.seg[0].K = op == SLIMKV_OP_LATENT ? C_K : wsb + pl.off_kb;
    a.seg[0].V = op == SLIMKV_OP_LATENT ? C_V : wsb + pl.off_vb;
  }
  if (raw) {
    a.seg[1].K = K_raw;
    a.seg[1].V = V_raw;
  }

  hipError_t err = hipSuccess;
  if ((p->flags & SLIMKV_FLAG_CHECK_WORKSPACE) && !noalloc)
    err = launch_workspace_check(reinterpret_cast<uint32_t*>(wsb), pl.off_counters, pl.off_ml, s);
  if (err == hipSuccess && op == SLIMKV_OP_RECONSTRUCT && beacons) {
    RebuildArgs rb{};
    rb.batch = p->batch;
    rb.num_kv_heads = p->num_kv_heads;
    rb.num_beacons = p->num_beacons;
    rb.C[0] = C_K;
    rb.U[0] = U_K;
    rb.dst[0] = wsb + pl.off_kb;
    rb.rank[0] = (int32_t)rk;
    rb.C[1] = C_V;
    rb.U[1] = U_V;
    rb.dst[1] = wsb + pl.off_vb;
    rb.rank[1] = (int32_t)rv;
    rb.pos = beacon_pos;  // keys only
    for (int k = 0; k < 6; ++k) rb.inv_freq_pow2[k] = a.inv_freq_pow2[k];
    err = launch_rebuild(rb, pl.dtype, s);
  }
  if (err == hipSuccess) {
    const hipEvent_t ev0 = g_ev_start, ev1 = g_ev_stop;
    g_ev_start = g_ev_stop = nullptr;
    err = launch_attention(a, pl.dtype, s, ev0, ev1);
  }
  if (err != hipSuccess) return fail(SLIMKV_ERR_HIP, "HIP launch failed: %s", hipGetErrorString(err));
  g_last_error.clear();
  return SLIMKV_OK;
}

// Page-table checks of a paged call: the page size, the table widths
// against the capacities and the on-chip table limit.  Sets *shift to
// log2(page_rows) and pool_bytes to the sizes of the C_K, C_V, K_raw and
// V_raw pools.
slimkv_status check_pages(const slimkv_problem* p, const slimkv_pages* pg, int elem, int* shift,
                          size_t pool_bytes[4]) {
  if (!pg) return fail(SLIMKV_ERR_NULL, "pages is NULL");
  const int pr = pg->page_rows;
  if (pr < (1 << kMinPageShift) || pr > (1 << kMaxPageShift) || (pr & (pr - 1)) != 0)
    return fail(SLIMKV_ERR_SHAPE, "page_rows %d is not a power of two in [%d, %d]", pr,
                1 << kMinPageShift, 1 << kMaxPageShift);
  if (pg->reserved != 0) return fail(SLIMKV_ERR_SHAPE, "pages->reserved must be 0");
  *shift = __builtin_ctz((unsigned)pr);
  const int64_t nbp = ceil_div(p->num_beacons, pr), nrp = ceil_div(p->raw_window, pr);
  if (nbp + nrp > kMaxPageEntries)
    return fail(SLIMKV_ERR_UNSUPPORTED, "%lld + %lld pages per sequence exceed %d",
                (long long)nbp, (long long)nrp, kMaxPageEntries);
  const struct {
    int64_t need;
    int32_t width, pages;
    const int32_t* table;
    const char* name;
  } seg[2] = {{nbp, pg->beacon_table_width, pg->beacon_pages, pg->beacon_table, "beacon"},
              {nrp, pg->raw_table_width, pg->raw_pages, pg->raw_table, "raw"}};
  for (const auto& sg : seg) {
    if (sg.need == 0) continue;
    if (!sg.table) return fail(SLIMKV_ERR_NULL, "%s_table is NULL", sg.name);
    if ((uintptr_t)sg.table % 4 != 0)
      return fail(SLIMKV_ERR_ALIGN, "%s_table is not 4-byte aligned", sg.name);
    if (sg.width < sg.need)
      return fail(SLIMKV_ERR_SHAPE, "%s_table_width %d is below the %lld pages of the capacity",
                  sg.name, sg.width, (long long)sg.need);
    if (sg.pages < 1) return fail(SLIMKV_ERR_SHAPE, "%s_pages must be >= 1", sg.name);
  }
  // pool bytes: pages x H_kv x page_rows x width x elem, for C_K, C_V, K_raw, V_raw
  const int64_t widths[4] = {p->num_beacons > 0 ? p->rank_k : 0, p->num_beacons > 0 ? p->rank_v : 0,
                             kHeadDim, kHeadDim};
  for (int i = 0; i < 4; ++i) {
    const auto& sg = seg[i / 2];
    const double bytes = (double)sg.pages * p->num_kv_heads * pr * widths[i] * elem;
    if (sg.need > 0 && bytes > 4.0e18)
      return fail(SLIMKV_ERR_SHAPE, "the %s pools are too large", sg.name);
    pool_bytes[i] = sg.need > 0 ? (size_t)sg.pages * p->num_kv_heads * pr * widths[i] * elem : 0;
  }
  return SLIMKV_OK;
}

// The ragged and paged calls (chunk = 0) and the chunk call (chunk = Q
// query tokens per sequence: q, out, lse, k_new and v_new carry a token axis).
slimkv_status run_ragged(const slimkv_problem* p, const slimkv_pages* pg, const void* q,
                         const int32_t* q_pos, const void* U_K, const void* U_V, const void* C_K,
                         const void* C_V, void* K_raw, void* V_raw, const int32_t* seq_beacons,
                         const int32_t* seq_raw, const void* k_new, const void* v_new, float* out,
                         float* lse, void* ws, size_t ws_bytes, void* stream, bool paged,
                         int32_t chunk = 0, const Alibi& alibi = Alibi()) {
  Plan pl;
  slimkv_status st = chunk > 0 ? make_chunk_plan(p, chunk, pl)
                               : make_plan(p, SLIMKV_OP_LATENT_RAGGED, pl);
  if (st != SLIMKV_OK) return st;
  st = check_alibi(p, alibi);
  if (st != SLIMKV_OK) return st;
  const size_t e = (size_t)pl.elem;
  const size_t T = chunk > 0 ? (size_t)chunk : 1;  // query tokens per sequence
  const size_t B = p->batch, Hq = p->num_q_heads, Hkv = p->num_kv_heads, d = kHeadDim;
  const size_t nb = p->num_beacons, w = p->raw_window;
  const bool beacons = nb > 0, raw = w > 0, append = k_new != nullptr || v_new != nullptr;
  const size_t rk = beacons ? p->rank_k : 0, rv = beacons ? p->rank_v : 0;
  // bytes of C_K, C_V, K_raw, V_raw: capacity arrays, or page pools
  size_t cache_bytes[4] = {B * Hkv * nb * rk * e, B * Hkv * nb * rv * e, B * Hkv * w * d * e,
                           B * Hkv * w * d * e};
  int shift = 0;
  if (paged) {
    st = check_pages(p, pg, pl.elem, &shift, cache_bytes);
    if (st != SLIMKV_OK) return st;
  }
  if (append && (!k_new || !v_new)) return fail(SLIMKV_ERR_NULL, "k_new and v_new go together");

  // Inputs read as 16-byte vectors, then the int32 ones; with a new token
  // the raw arrays are also written, so they count as outputs too.
  const bool btab = paged && beacons, rtab = paged && raw;
  Range in[12] = {
      {q, T * B * Hq * d * e, "q"},
      {beacons ? U_K : nullptr, Hkv * d * rk * e, "U_K"},
      {beacons ? U_V : nullptr, Hkv * d * rv * e, "U_V"},
      {beacons ? C_K : nullptr, cache_bytes[0], "C_K"},
      {beacons ? C_V : nullptr, cache_bytes[1], "C_V"},
      {append ? k_new : nullptr, T * B * Hkv * d * e, "k_new"},
      {append ? v_new : nullptr, T * B * Hkv * d * e, "v_new"},
      {q_pos, B * sizeof(int32_t), "q_pos"},
      {seq_beacons, seq_beacons ? B * sizeof(int32_t) : 0, "num_beacons_b"},
      {seq_raw, seq_raw ? B * sizeof(int32_t) : 0, "raw_len"},
      {btab ? pg->beacon_table : nullptr, btab ? B * pg->beacon_table_width * sizeof(int32_t) : 0,
       "beacon_table"},
      {rtab ? pg->raw_table : nullptr, rtab ? B * pg->raw_table_width * sizeof(int32_t) : 0,
       "raw_table"},
  };
  const Range kr{raw ? K_raw : nullptr, cache_bytes[2], "K_raw"};
  const Range vr{raw ? V_raw : nullptr, cache_bytes[3], "V_raw"};
  Range req[11];
  int n_req = 0;
  req[n_req++] = in[0];
  req[n_req++] = in[7];
  if (beacons)
    for (int i = 1; i < 5; ++i) req[n_req++] = in[i];
  if (raw) {
    req[n_req++] = kr;
    req[n_req++] = vr;
  }
  req[n_req++] = Range{out, 1, "out"};
  Range outs[5] = {{out, T * B * Hq * d * sizeof(float), "out"},
                   {lse, lse ? T * B * Hq * sizeof(float) : 0, "lse"},
                   {ws, pl.total, "workspace"},
                   {append ? kr.p : nullptr, append ? kr.bytes : 0, "K_raw"},
                   {append ? vr.p : nullptr, append ? vr.bytes : 0, "V_raw"}};
  Range all_in[14];
  int n_in = 0;
  for (int i = 0; i < 12; ++i) all_in[n_in++] = in[i];
  if (!append) {
    all_in[n_in++] = kr;
    all_in[n_in++] = vr;
  }
  for (int i = 7; i < 10; ++i)
    if (in[i].p && (uintptr_t)in[i].p % 4 != 0)
      return fail(SLIMKV_ERR_ALIGN, "%s is not 4-byte aligned", in[i].name);
  for (const Range* x : {&kr, &vr})
    if (x->p && (uintptr_t)x->p % 16 != 0)
      return fail(SLIMKV_ERR_ALIGN, "%s is not 16-byte aligned", x->name);
  if (alibi.slopes) {
    const Range sl{alibi.slopes, Hq * sizeof(float), "slopes"};
    for (const Range& o : outs)
      if (overlap(o, sl)) return fail(SLIMKV_ERR_ALIAS, "%s overlaps slopes", o.name);
  }
  st = check_pointers(in, 7, req, n_req, outs, 0, 16);  // presence and 16-byte alignment
  if (st != SLIMKV_OK) return st;
  st = check_pointers(all_in, n_in, req, 0, outs, 5, 1);  // overlaps
  if (st != SLIMKV_OK) return st;
  if (!ws) return fail(SLIMKV_ERR_NULL, "workspace is NULL");
  if ((uintptr_t)ws % 16 != 0) return fail(SLIMKV_ERR_ALIGN, "workspace is not 16-byte aligned");
  if (ws_bytes < pl.total)
    return fail(SLIMKV_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, pl.total);

  char* wsb = static_cast<char*>(ws);
  AttnArgs& a = pl.attn;
  a.q = q;
  a.q_pos = q_pos;
  a.U_K = U_K;
  a.U_V = U_V;
  for (int k = 0; k < 6; ++k)
    a.inv_freq_pow2[k] = pow(p->rope_theta, -2.0 * (double)(1 << k) / (double)kHeadDim);
  a.score_scale = (double)p->scale * 1.4426950408889634074;
  a.counters = reinterpret_cast<uint32_t*>(wsb + pl.off_counters);
  a.flags = reinterpret_cast<uint32_t*>(wsb + pl.off_flags);
  a.part_ml = reinterpret_cast<float*>(wsb + pl.off_ml);
  a.part_acc = reinterpret_cast<float*>(wsb + pl.off_acc);
  a.out = out;
  a.lse = lse;
  if (beacons) {
    a.seg[0].K = C_K;
    a.seg[0].V = C_V;
  }
  if (raw) {
    a.seg[1].K = K_raw;
    a.seg[1].V = V_raw;
  }
  a.seq_beacons = seq_beacons;
  a.seq_raw = seq_raw;
  a.alibi_slopes = alibi.slopes;
  a.beacon_first = alibi.first;
  a.beacon_stride = alibi.stride;
  a.k_new = append ? k_new : nullptr;
  a.v_new = append ? v_new : nullptr;
  a.k_store = K_raw;
  a.v_store = V_raw;
  // unit u's new-token partial takes the slot after all pieces' (ragged:
  // pieces below units * kMaxChunks of units * (kMaxChunks + 1) slots;
  // chunk: below units + kChunkMaxSlots of 2 units + kChunkMaxSlots)
  a.tok_slot0 = (int32_t)(chunk > 0 ? pl.units + kChunkMaxSlots : pl.units * kMaxChunks);
  if (paged) {
    a.page_table[0] = btab ? pg->beacon_table : nullptr;
    a.page_table[1] = rtab ? pg->raw_table : nullptr;
    a.table_width[0] = pg->beacon_table_width;
    a.table_width[1] = pg->raw_table_width;
    a.num_pages[0] = pg->beacon_pages;
    a.num_pages[1] = pg->raw_pages;
    a.page_shift = shift;
  }
  a.deterministic = 1;
  if (p->flags & SLIMKV_FLAG_CHECK_WORKSPACE) {
    const hipError_t e = launch_workspace_check(reinterpret_cast<uint32_t*>(wsb), pl.off_counters,
                                                pl.off_ml, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(SLIMKV_ERR_HIP, "HIP launch failed: %s", hipGetErrorString(e));
  }
  const hipEvent_t ev0 = g_ev_start, ev1 = g_ev_stop;
  g_ev_start = g_ev_stop = nullptr;
  const hipError_t err = chunk > 0
                            ? launch_chunk(a, pl.dtype, static_cast<hipStream_t>(stream), ev0, ev1)
                            : launch_ragged(a, pl.dtype, static_cast<hipStream_t>(stream), ev0, ev1);
  if (err != hipSuccess) return fail(SLIMKV_ERR_HIP, "HIP launch failed: %s", hipGetErrorString(err));
  g_last_error.clear();
  return SLIMKV_OK;
}

}  // namespace
}  // namespace slimkv

extern "C" {

size_t slimkv_workspace_bytes(const slimkv_problem* problem, slimkv_op op) {
  slimkv::Plan pl;
  if (slimkv::make_plan(problem, op, pl) != SLIMKV_OK) return 0;
  return pl.total;
}

slimkv_status slimkv_decode_attn(const slimkv_problem* problem, const void* q, const int32_t* q_pos,
                                 const void* U_K, const void* U_V, const void* C_K, const void* C_V,
                                 const void* K_raw, const void* V_raw, float* out, float* lse,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  return slimkv::run(problem, SLIMKV_OP_LATENT, q, q_pos, U_K, U_V, C_K, C_V, K_raw, V_raw, out,
                     lse, workspace, workspace_bytes, stream);
}

slimkv_status slimkv_decode_attn_noalloc(const slimkv_problem* problem, const void* q,
                                         const int32_t* q_pos, const void* U_K, const void* U_V,
                                         const void* C_K, const void* C_V, const void* K_raw,
                                         const void* V_raw, float* out, float* lse, void* stream) {
  return slimkv::run(problem, SLIMKV_OP_LATENT, q, q_pos, U_K, U_V, C_K, C_V, K_raw, V_raw, out,
                     lse, nullptr, 0, stream, nullptr, slimkv::Alibi(), true);
}

slimkv_status slimkv_reconstruct_attn(const slimkv_problem* problem, const void* q,
                                      const int32_t* q_pos, const void* U_K, const void* U_V,
                                      const void* C_K, const void* C_V, const void* K_raw,
                                      const void* V_raw, float* out, float* lse, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  return slimkv::run(problem, SLIMKV_OP_RECONSTRUCT, q, q_pos, U_K, U_V, C_K, C_V, K_raw, V_raw,
                     out, lse, workspace, workspace_bytes, stream);
}

slimkv_status slimkv_reconstruct_rope_attn(const slimkv_problem* problem, const void* q,
                                           const int32_t* q_pos, const void* U_K, const void* U_V,
                                           const void* C_K, const void* C_V, const void* K_raw,
                                           const void* V_raw, const int32_t* beacon_pos, float* out,
                                           float* lse, void* workspace, size_t workspace_bytes,
                                           void* stream) {
  if (problem && problem->num_beacons > 0 && !beacon_pos)
    return slimkv::fail(SLIMKV_ERR_NULL, "beacon_pos is NULL");
  return slimkv::run(problem, SLIMKV_OP_RECONSTRUCT, q, q_pos, U_K, U_V, C_K, C_V, K_raw, V_raw,
                     out, lse, workspace, workspace_bytes, stream, beacon_pos);
}

slimkv_status full_kv_attn(const slimkv_problem* problem, const void* q, const int32_t* q_pos,
                           const void* K, const void* V, float* out, float* lse, void* workspace,
                           size_t workspace_bytes, void* stream) {
  return slimkv::run(problem, SLIMKV_OP_FULL_KV, q, q_pos, nullptr, nullptr, nullptr, nullptr, K,
                     V, out, lse, workspace, workspace_bytes, stream);
}

slimkv_status slimkv_decode_attn_ragged(const slimkv_problem* problem, const void* q,
                                        const int32_t* q_pos, const void* U_K, const void* U_V,
                                        const void* C_K, const void* C_V, void* K_raw, void* V_raw,
                                        const int32_t* num_beacons_b, const int32_t* raw_len,
                                        const void* k_new, const void* v_new, float* out, float* lse,
                                        void* workspace, size_t workspace_bytes, void* stream) {
  return slimkv::run_ragged(problem, nullptr, q, q_pos, U_K, U_V, C_K, C_V, K_raw, V_raw,
                            num_beacons_b, raw_len, k_new, v_new, out, lse, workspace,
                            workspace_bytes, stream, false);
}

slimkv_status slimkv_decode_attn_paged(const slimkv_problem* problem, const slimkv_pages* pages,
                                       const void* q, const int32_t* q_pos, const void* U_K,
                                       const void* U_V, const void* C_K, const void* C_V,
                                       void* K_raw, void* V_raw, const int32_t* num_beacons_b,
                                       const int32_t* raw_len, const void* k_new,
                                       const void* v_new, float* out, float* lse, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  return slimkv::run_ragged(problem, pages, q, q_pos, U_K, U_V, C_K, C_V, K_raw, V_raw,
                            num_beacons_b, raw_len, k_new, v_new, out, lse, workspace,
                            workspace_bytes, stream, true);
}

slimkv_status slimkv_decode_attn_alibi(const slimkv_problem* problem, const void* q,
                                       const int32_t* q_pos, const void* U_K, const void* U_V,
                                       const void* C_K, const void* C_V, const void* K_raw,
                                       const void* V_raw, const float* slopes,
                                       int32_t beacon_first, int32_t beacon_stride, float* out,
                                       float* lse, void* workspace, size_t workspace_bytes,
                                       void* stream) {
  if (!slopes) return slimkv::fail(SLIMKV_ERR_NULL, "slopes is NULL");
  slimkv::Alibi al;
  al.slopes = slopes;
  al.first = beacon_first;
  al.stride = beacon_stride;
  return slimkv::run(problem, SLIMKV_OP_LATENT, q, q_pos, U_K, U_V, C_K, C_V, K_raw, V_raw, out,
                     lse, workspace, workspace_bytes, stream, nullptr, al);
}

static slimkv::Alibi alibi_of(const slimkv_alibi* al) {
  slimkv::Alibi r;
  r.slopes = al->slopes;
  r.first = al->beacon_first;
  r.stride = al->beacon_stride;
  return r;
}

slimkv_status slimkv_decode_attn_ragged_alibi(const slimkv_problem* problem,
                                              const slimkv_alibi* alibi, const void* q,
                                              const int32_t* q_pos, const void* U_K,
                                              const void* U_V, const void* C_K, const void* C_V,
                                              void* K_raw, void* V_raw,
                                              const int32_t* num_beacons_b, const int32_t* raw_len,
                                              const void* k_new, const void* v_new, float* out,
                                              float* lse, void* workspace, size_t workspace_bytes,
                                              void* stream) {
  if (!alibi || !alibi->slopes) return slimkv::fail(SLIMKV_ERR_NULL, "alibi or its slopes is NULL");
  return slimkv::run_ragged(problem, nullptr, q, q_pos, U_K, U_V, C_K, C_V, K_raw, V_raw,
                            num_beacons_b, raw_len, k_new, v_new, out, lse, workspace,
                            workspace_bytes, stream, false, 0, alibi_of(alibi));
}

slimkv_status slimkv_decode_attn_paged_alibi(const slimkv_problem* problem,
                                             const slimkv_pages* pages, const slimkv_alibi* alibi,
                                             const void* q, const int32_t* q_pos, const void* U_K,
                                             const void* U_V, const void* C_K, const void* C_V,
                                             void* K_raw, void* V_raw,
                                             const int32_t* num_beacons_b, const int32_t* raw_len,
                                             const void* k_new, const void* v_new, float* out,
                                             float* lse, void* workspace, size_t workspace_bytes,
                                             void* stream) {
  if (!alibi || !alibi->slopes) return slimkv::fail(SLIMKV_ERR_NULL, "alibi or its slopes is NULL");
  return slimkv::run_ragged(problem, pages, q, q_pos, U_K, U_V, C_K, C_V, K_raw, V_raw,
                            num_beacons_b, raw_len, k_new, v_new, out, lse, workspace,
                            workspace_bytes, stream, true, 0, alibi_of(alibi));
}

slimkv_status slimkv_decode_attn_chunk_alibi(const slimkv_problem* problem,
                                             const slimkv_alibi* alibi, int32_t num_tokens,
                                             const void* q, const int32_t* q_pos, const void* U_K,
                                             const void* U_V, const void* C_K, const void* C_V,
                                             void* K_raw, void* V_raw,
                                             const int32_t* num_beacons_b, const int32_t* raw_len,
                                             const void* k_new, const void* v_new, float* out,
                                             float* lse, void* workspace, size_t workspace_bytes,
                                             void* stream) {
  if (!alibi || !alibi->slopes) return slimkv::fail(SLIMKV_ERR_NULL, "alibi or its slopes is NULL");
  if (num_tokens < 1) return slimkv::fail(SLIMKV_ERR_SHAPE, "num_tokens must be >= 1");
  return slimkv::run_ragged(problem, nullptr, q, q_pos, U_K, U_V, C_K, C_V, K_raw, V_raw,
                            num_beacons_b, raw_len, k_new, v_new, out, lse, workspace,
                            workspace_bytes, stream, false, num_tokens, alibi_of(alibi));
}

slimkv_status slimkv_decode_attn_chunk_paged_alibi(
    const slimkv_problem* problem, const slimkv_pages* pages, const slimkv_alibi* alibi,
    int32_t num_tokens, const void* q, const int32_t* q_pos, const void* U_K, const void* U_V,
    const void* C_K, const void* C_V, void* K_raw, void* V_raw, const int32_t* num_beacons_b,
    const int32_t* raw_len, const void* k_new, const void* v_new, float* out, float* lse,
    void* workspace, size_t workspace_bytes, void* stream) {
  if (!alibi || !alibi->slopes) return slimkv::fail(SLIMKV_ERR_NULL, "alibi or its slopes is NULL");
  if (num_tokens < 1) return slimkv::fail(SLIMKV_ERR_SHAPE, "num_tokens must be >= 1");
  return slimkv::run_ragged(problem, pages, q, q_pos, U_K, U_V, C_K, C_V, K_raw, V_raw,
                            num_beacons_b, raw_len, k_new, v_new, out, lse, workspace,
                            workspace_bytes, stream, true, num_tokens, alibi_of(alibi));
}

size_t slimkv_chunk_workspace_bytes(const slimkv_problem* problem, int32_t num_tokens) {
  slimkv::Plan pl;
  if (slimkv::make_chunk_plan(problem, num_tokens, pl) != SLIMKV_OK) return 0;
  return pl.total;
}

slimkv_status slimkv_decode_attn_chunk(const slimkv_problem* problem, int32_t num_tokens,
                                       const void* q, const int32_t* q_pos, const void* U_K,
                                       const void* U_V, const void* C_K, const void* C_V,
                                       void* K_raw, void* V_raw, const int32_t* num_beacons_b,
                                       const int32_t* raw_len, const void* k_new,
                                       const void* v_new, float* out, float* lse, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  if (num_tokens < 1) return slimkv::fail(SLIMKV_ERR_SHAPE, "num_tokens must be >= 1");
  return slimkv::run_ragged(problem, nullptr, q, q_pos, U_K, U_V, C_K, C_V, K_raw, V_raw,
                            num_beacons_b, raw_len, k_new, v_new, out, lse, workspace,
                            workspace_bytes, stream, false, num_tokens);
}

slimkv_status slimkv_decode_attn_chunk_paged(const slimkv_problem* problem,
                                             const slimkv_pages* pages, int32_t num_tokens,
                                             const void* q, const int32_t* q_pos, const void* U_K,
                                             const void* U_V, const void* C_K, const void* C_V,
                                             void* K_raw, void* V_raw,
                                             const int32_t* num_beacons_b, const int32_t* raw_len,
                                             const void* k_new, const void* v_new, float* out,
                                             float* lse, void* workspace, size_t workspace_bytes,
                                             void* stream) {
  if (num_tokens < 1) return slimkv::fail(SLIMKV_ERR_SHAPE, "num_tokens must be >= 1");
  return slimkv::run_ragged(problem, pages, q, q_pos, U_K, U_V, C_K, C_V, K_raw, V_raw,
                            num_beacons_b, raw_len, k_new, v_new, out, lse, workspace,
                            workspace_bytes, stream, true, num_tokens);
}

const char* slimkv_status_string(slimkv_status status) {
  switch (status) {
    case SLIMKV_OK: return "ok";
    case SLIMKV_ERR_NULL: return "a required pointer is NULL";
    case SLIMKV_ERR_SHAPE: return "inconsistent or out-of-range sizes";
    case SLIMKV_ERR_UNSUPPORTED: return "valid but unsupported problem";
    case SLIMKV_ERR_WORKSPACE: return "workspace too small";
    case SLIMKV_ERR_ALIGN: return "misaligned device pointer";
    case SLIMKV_ERR_ALIAS: return "an output overlaps an input or another output";
    case SLIMKV_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

const char* slimkv_last_error(void) { return slimkv::g_last_error.c_str(); }

slimkv_status slimkv_set_kernel_events(void* start, void* stop) {
  if ((start == nullptr) != (stop == nullptr))
    return slimkv::fail(SLIMKV_ERR_NULL, "start and stop must both be set or both be NULL");
  slimkv::g_ev_start = static_cast<hipEvent_t>(start);
  slimkv::g_ev_stop = static_cast<hipEvent_t>(stop);
  return SLIMKV_OK;
}

int32_t slimkv_abi_version(void) { return SLIMKV_ABI_VERSION; }

slimkv_status slimkv_workspace_status(const void* workspace, uint32_t* status) {
  if (!workspace || !status) return slimkv::fail(SLIMKV_ERR_NULL, "workspace or status is NULL");
  if ((uintptr_t)workspace % 16 != 0)
    return slimkv::fail(SLIMKV_ERR_ALIGN, "workspace is not 16-byte aligned");
  const hipError_t e = hipMemcpy(status, workspace, sizeof(uint32_t), hipMemcpyDeviceToHost);
  if (e != hipSuccess)
    return slimkv::fail(SLIMKV_ERR_HIP, "reading the status word failed: %s", hipGetErrorString(e));
  return SLIMKV_OK;
}

}  // extern "C"
