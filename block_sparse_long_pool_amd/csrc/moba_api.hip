// Host side of libmoba: argument checks, workspace layouts and launch sequences of the
// MoBA prefill forward (batched and packed), its backward, the dense causal and decode
// paths, the key convolution and the stage entry points.  Every check runs before the
// first launch.
#include <math.h>
#include <string.h>

#include <mutex>

#include "../../include/moba.h"
#include "moba_internal.h"

using moba::Shape;

namespace {

constexpr size_t kAlign = 256;
// The gate's rank keys keep 23 - ceil(log2 nb) mantissa bits of a score: at 8192 blocks
// that is 10 bits, a resolution below the 1e-3-relative near-tie band.
constexpr int kMaxBlocks = 8192;

size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

// topk >= the number of blocks of the longest sequence: every row selects every causal
// block, so the layer is dense causal attention (README bullet "Seamlessly Transition
// between Full and Sparse Attention").  That case runs as one block of the whole
// sequence, with no gate, index or history partials.
bool all_blocks(int seqlen, int block, int topk) { return (long long)topk * block >= seqlen; }
bool all_blocks(const Shape& s) { return all_blocks(s.T, s.block, s.topk); }

// the dense causal form of a shape: one block of the whole (longest) sequence, top-1
Shape dense_shape(const Shape& s) {
  Shape d = s;
  d.block = (s.T + 15) / 16 * 16;
  d.topk = 1;
  return d;
}

int check(int batch, int seqlen, int hq, int hkv, int head_dim, int block, int topk,
          float scale) {
  if (batch <= 0 || seqlen <= 0 || hq <= 0 || hkv <= 0 || head_dim <= 0 || block <= 0 ||
      topk <= 0)
    return MOBA_ERR_INVALID_ARG;
  if (hq % hkv != 0) return MOBA_ERR_INVALID_ARG;
  if (!isfinite(scale)) return MOBA_ERR_INVALID_ARG;
  if (scale <= 0.f) return MOBA_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return MOBA_ERR_UNSUPPORTED;
  if (block < 16 || block % 16 != 0) return MOBA_ERR_UNSUPPORTED;
  if ((long long)batch * seqlen * hq >= (1ll << 31)) return MOBA_ERR_UNSUPPORTED;
  if (all_blocks(seqlen, block, topk)) return MOBA_OK;
  // sparse: topk - 1 history slots ranked by the gate, index rows of 32 - sbits bits
  if (topk - 1 > moba::gate_max_history()) return MOBA_ERR_UNSUPPORTED;
  if ((seqlen + block - 1) / block > kMaxBlocks) return MOBA_ERR_UNSUPPORTED;
  const long long G = hq / hkv;
  if ((long long)seqlen * G >= (1ll << (32 - moba::entry_slot_bits(topk))))
    return MOBA_ERR_UNSUPPORTED;
  return MOBA_OK;
}

// rows of one query head of one sequence that carry history slot entries, times slots
// (a partial last block has fewer rows)
long long entries_per_head(const Shape& s) {
  long long per = 0;
  for (int c = 0; c < s.nb(); ++c) {
    const int rows = s.T - c * s.block < s.block ? s.T - c * s.block : s.block;
    per += (long long)rows * (c < s.KH() ? c : s.KH());
  }
  return per;
}

// entries of a group of ng kv-heads: exact for a uniform batch; for packed sequences a
// bound (every token with every slot), since the lengths live on the device
long long group_entries(const Shape& s, int ng) {
  if (s.cu) return (long long)ng * s.G() * s.total * s.KH();
  return (long long)s.b * ng * s.G() * entries_per_head(s);
}

// rows of the history partials of a group of ng kv-heads
size_t group_part_rows(const Shape& s, int ng) {
  const size_t tokens = s.cu ? (size_t)s.total : (size_t)s.b * s.T;
  return tokens * ng * s.G() * s.KH();
}

struct Layout {
  // whole-problem buffers
  size_t pool_partial, cent, chi, clo;
  // per group of ng kv-heads
  size_t chunk_counts, list_count, list_offsets, tile_offsets, tiles, entries, part_o,
      part_lse;
  size_t total;
  long long n_entries;
  long long max_tiles;
  int tile_rows;               // rows per history-attention tile
};

// tile_rows 0: the history tile length for this group size; else the given one (every
// pass of a forward uses the first group's, for which the tile buffer is sized)
Layout make_layout(const Shape& s, int ng, int tile_rows = 0) {
  Layout L{};
  const size_t nb = s.nb();
  const size_t splits = moba::pool_splits(s);
  const size_t ncent = (size_t)s.b * s.hkv * nb * s.d;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  L.pool_partial = take((size_t)s.b * nb * splits * s.hkv * s.d * sizeof(float));
  L.cent = take(ncent * sizeof(float));
  L.chi = take(ncent * sizeof(uint16_t));
  L.clo = take(ncent * sizeof(uint16_t));
  const size_t nlists = (size_t)s.b * ng * nb;
  const size_t nchunks = moba::index_chunks(s);
  L.n_entries = group_entries(s, ng);
  L.tile_rows = tile_rows > 0 ? tile_rows : moba::history_tile_rows(s, L.n_entries);
  const int tm = L.tile_rows;
  L.max_tiles = (L.n_entries + tm - 1) / tm + (long long)nlists;
  L.chunk_counts = take((size_t)s.b * ng * nchunks * nb * sizeof(int32_t));
  L.list_count = take(nlists * sizeof(int32_t));
  L.list_offsets = take((nlists + 1) * sizeof(int32_t));
  L.tile_offsets = take((nlists + 2) * sizeof(int32_t));   // + count + queue counter
  L.tiles = take((size_t)L.max_tiles * sizeof(int4));
  L.entries = take((size_t)L.n_entries * sizeof(uint32_t));
  const size_t prow = group_part_rows(s, ng);   // history slots only
  L.part_o = take(prow * s.d * sizeof(uint16_t));   // bf16 partial outputs
  L.part_lse = take(prow * sizeof(float));          // fp32, slot-major [k-1][rows]
  L.total = off;
  return L;
}

bool layout_ok(const Layout& L) {
  return L.n_entries < (1ll << 31) && L.max_tiles < (1ll << 31);
}

// Backward workspace: D for the whole problem, then per group of ng kv-heads the
// inverted index (as in the forward, cut in tiles of the dQ kernel's rows) and the
// fp32 dQ parts of every (row, history slot).
struct BwdLayout {
  size_t delta, chunk_counts, list_count, list_offsets, tile_offsets, tiles, entries,
      dense_rows, dense_meta, dq_part;
  size_t total;
  long long n_entries, max_tiles;
};

BwdLayout make_bwd_layout(const Shape& s, int ng) {
  BwdLayout L{};
  const size_t nb = s.nb();
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  const size_t tokens = s.cu ? (size_t)s.total : (size_t)s.b * s.T;
  L.delta = take(tokens * s.hq * sizeof(float));
  const size_t nlists = (size_t)s.b * ng * nb;
  const size_t nchunks = moba::index_chunks(s);
  L.n_entries = group_entries(s, ng);
  const int tm = moba::bwd_tile_rows();
  L.max_tiles = (L.n_entries + tm - 1) / tm + (long long)nlists;
  L.chunk_counts = take((size_t)s.b * ng * nchunks * nb * sizeof(int32_t));
  L.list_count = take(nlists * sizeof(int32_t));
  L.list_offsets = take((nlists + 1) * sizeof(int32_t));
  L.tile_offsets = take((nlists + 2) * sizeof(int32_t));   // + count + queue counter
  L.tiles = take((size_t)L.max_tiles * sizeof(int4));
  L.entries = take((size_t)L.n_entries * sizeof(uint32_t));
  L.dense_rows = take((size_t)L.n_entries * 2 * s.d * sizeof(uint16_t));
  L.dense_meta = take((size_t)L.n_entries * 2 * sizeof(float));
  L.dq_part = take(group_part_rows(s, ng) * s.d * sizeof(float));
  L.total = off;
  return L;
}

bool bwd_layout_ok(const BwdLayout& L) {
  return L.n_entries < (1ll << 31) && L.max_tiles < (1ll << 31);
}

int hip_status(hipError_t e) { return e == hipSuccess ? MOBA_OK : MOBA_ERR_HIP; }

#define MOBA_TRY(expr)                        \
  do {                                        \
    hipError_t _e = (expr);                   \
    if (_e != hipSuccess) return MOBA_ERR_HIP; \
  } while (0)

}  // namespace

extern "C" {

int moba_check_args(int batch, int seqlen, int hq, int hkv, int head_dim, int block,
                    int topk, float scale) {
  return check(batch, seqlen, hq, hkv, head_dim, block, topk, scale);
}

size_t moba_workspace_bytes(int batch, int seqlen, int hq, int hkv, int head_dim,
                            int block, int topk, size_t* min_bytes) {
  if (min_bytes) *min_bytes = 0;
  if (check(batch, seqlen, hq, hkv, head_dim, block, topk, 1.f) != MOBA_OK) return 0;
  const Shape s{batch, seqlen, hq, hkv, head_dim, block, topk};
  if (all_blocks(s)) {          // dense causal: no workspace is used
    if (min_bytes) *min_bytes = kAlign;
    return kAlign;
  }
  const Layout one = make_layout(s, 1);
  if (!layout_ok(one)) return 0;
  if (min_bytes) *min_bytes = one.total;
  for (int ng = hkv; ng >= 1; --ng) {
    const Layout L = make_layout(s, ng);
    if (layout_ok(L)) return L.total;
  }
  return one.total;
}

const char* moba_strerror(int status) {
  switch (status) {
    case MOBA_OK: return "success";
    case MOBA_ERR_INVALID_ARG: return "invalid argument";
    case MOBA_ERR_UNSUPPORTED: return "shape or value not supported by this library";
    case MOBA_ERR_WORKSPACE: return "workspace too small";
    case MOBA_ERR_HIP: return "HIP launch or runtime error";
    default: return "unknown status";
  }
}

}  // extern "C"

namespace {

// Records HIP events at stage boundaries on the launch stream when profiling.
// Stage boundaries as HIP events on the launch stream.  Either the clock owns its
// events and sums the stage times at the end (synchronising), or the caller gives
// MOBA_NUM_STAGES + 1 events that are only recorded: ext[0] at the start and
// ext[i + 1] after stage i (the last kv-head group's boundaries when there are several).
struct StageClock {
  hipStream_t st;
  bool on = false;
  hipEvent_t const* ext = nullptr;
  int n = 0;
  int stage[64];
  hipEvent_t ev[65];
  bool begin(hipStream_t s, bool enable, void* const* external) {
    st = s;
    if (external) {
      ext = reinterpret_cast<hipEvent_t const*>(external);
      return hipEventRecord(ext[0], st) == hipSuccess;
    }
    on = enable;
    if (!on) return true;
    for (int i = 0; i < 65; ++i)
      if (hipEventCreate(&ev[i]) != hipSuccess) return false;
    return hipEventRecord(ev[0], st) == hipSuccess;
  }
  hipError_t mark(int which) {
    if (ext) return hipEventRecord(ext[which + 1], st);
    if (!on || n >= 64) return hipSuccess;
    stage[n] = which;
    return hipEventRecord(ev[++n], st);
  }
  int finish(float* ms) {
    if (!on) return MOBA_OK;
    int status = MOBA_OK;
    if (hipEventSynchronize(ev[n]) != hipSuccess) status = MOBA_ERR_HIP;
    for (int i = 0; i < MOBA_NUM_STAGES; ++i) ms[i] = 0.f;
    for (int i = 0; i < n && status == MOBA_OK; ++i) {
      float t = 0.f;
      if (hipEventElapsedTime(&t, ev[i], ev[i + 1]) != hipSuccess) status = MOBA_ERR_HIP;
      ms[stage[i]] += t;
    }
    for (int i = 0; i < 65; ++i) (void)hipEventDestroy(ev[i]);
    return status;
  }
};

// the whole forward for a validated shape (a uniform batch or packed sequences)
int run_forward(const Shape& s, const void* q, const void* k, const void* v, float scale,
                void* out, float* lse, int32_t* idx, void* workspace,
                size_t workspace_bytes, void* stream, float* stage_ms,
                void* const* stage_events) {
  if (!q || !k || !v || !out || !lse || !idx || !workspace) return MOBA_ERR_INVALID_ARG;
  if (((uintptr_t)workspace & (kAlign - 1)) != 0) return MOBA_ERR_INVALID_ARG;
  hipStream_t hs0 = static_cast<hipStream_t>(stream);
  if (all_blocks(s)) {
    // every causal block selected: idx lists them all, and the current-block kernel over
    // one block of the whole sequence is the attention; pool, index and history steps
    // are empty
    StageClock clock;
    if (!clock.begin(hs0, stage_ms != nullptr, stage_events)) return MOBA_ERR_HIP;
    MOBA_TRY(clock.mark(0));
    MOBA_TRY(moba::launch_idx_all_blocks(s, idx, hs0));
    MOBA_TRY(clock.mark(1));
    MOBA_TRY(clock.mark(2));
    MOBA_TRY(clock.mark(3));
    MOBA_TRY(moba::launch_attn_current(dense_shape(s), static_cast<const uint16_t*>(q),
                                       static_cast<const uint16_t*>(k),
                                       static_cast<const uint16_t*>(v), scale, 0, s.hkv,
                                       nullptr, nullptr, static_cast<uint16_t*>(out), lse,
                                       hs0));
    MOBA_TRY(clock.mark(4));
    return clock.finish(stage_ms);
  }
  const int hkv = s.hkv;
  // the largest group of kv-heads whose buffers fit
  int ng = hkv;
  Layout L = make_layout(s, ng);
  while (ng > 1 && (L.total > workspace_bytes || !layout_ok(L))) L = make_layout(s, --ng);
  if (L.total > workspace_bytes) return MOBA_ERR_WORKSPACE;
  if (!layout_ok(L)) return MOBA_ERR_UNSUPPORTED;

  char* ws = static_cast<char*>(workspace);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const uint16_t* qb = static_cast<const uint16_t*>(q);
  const uint16_t* kb = static_cast<const uint16_t*>(k);
  const uint16_t* vb = static_cast<const uint16_t*>(v);
  float* cent = reinterpret_cast<float*>(ws + L.cent);
  uint16_t* chi = reinterpret_cast<uint16_t*>(ws + L.chi);
  uint16_t* clo = reinterpret_cast<uint16_t*>(ws + L.clo);
  StageClock clock;
  if (!clock.begin(hs, stage_ms != nullptr, stage_events)) return MOBA_ERR_HIP;

  MOBA_TRY(moba::launch_pool(s, kb, reinterpret_cast<float*>(ws + L.pool_partial), cent, chi,
                             clo, hs));
  MOBA_TRY(clock.mark(0));
  MOBA_TRY(moba::launch_gate(s, qb, chi, clo, idx, hs));
  MOBA_TRY(clock.mark(1));

  for (int g0 = 0; g0 < hkv; g0 += ng) {
    const int ngc = ng < hkv - g0 ? ng : hkv - g0;
    const int nlc = s.b * ngc * s.nb();
    uint16_t* po = reinterpret_cast<uint16_t*>(ws + L.part_o);
    float* pl = reinterpret_cast<float*>(ws + L.part_lse);
    if (s.KH() > 0) {
      int32_t* tile_offsets = reinterpret_cast<int32_t*>(ws + L.tile_offsets);
      int4* tiles = reinterpret_cast<int4*>(ws + L.tiles);
      uint32_t* entries = reinterpret_cast<uint32_t*>(ws + L.entries);
      const Layout Lc = make_layout(s, ngc, L.tile_rows);
      MOBA_TRY(moba::launch_index(s, idx, g0, ngc, L.tile_rows,
                                  reinterpret_cast<int32_t*>(ws + L.chunk_counts),
                                  reinterpret_cast<int32_t*>(ws + L.list_count),
                                  reinterpret_cast<int32_t*>(ws + L.list_offsets),
                                  tile_offsets, tiles, entries, L.n_entries, hs));
      MOBA_TRY(clock.mark(2));
      MOBA_TRY(moba::launch_attn_history(s, qb, kb, vb, scale, g0, ngc, tiles,
                                         tile_offsets + nlc, (int)Lc.max_tiles, entries,
                                         po, pl, hs));
      MOBA_TRY(clock.mark(3));
    } else {
      // no history slots: the index and history stages are empty, but their
      // boundaries are still recorded so that every stage time is well defined
      MOBA_TRY(clock.mark(2));
      MOBA_TRY(clock.mark(3));
    }
    MOBA_TRY(moba::launch_attn_current(s, qb, kb, vb, scale, g0, ngc, po, pl,
                                       static_cast<uint16_t*>(out), lse, hs));
    MOBA_TRY(clock.mark(4));
  }
  return clock.finish(stage_ms);
}

int forward_impl(const void* q, const void* k, const void* v, int batch, int seqlen,
                 int hq, int hkv, int head_dim, int block, int topk, float scale,
                 void* out, float* lse, int32_t* idx, void* workspace,
                 size_t workspace_bytes, void* stream, float* stage_ms,
                 void* const* stage_events) {
  const int st = check(batch, seqlen, hq, hkv, head_dim, block, topk, scale);
  if (st != MOBA_OK) return st;
  const Shape s{batch, seqlen, hq, hkv, head_dim, block, topk};
  return run_forward(s, q, k, v, scale, out, lse, idx, workspace, workspace_bytes, stream,
                     stage_ms, stage_events);
}

// packed sequences: the shape checks of a batch of nseq sequences of max_seqlen tokens,
// plus the packed token count
int varlen_shape(int nseq, int total, int max_seqlen, int hq, int hkv, int head_dim,
                 int block, int topk, float scale, const int32_t* cu, Shape* out) {
  const int st = check(nseq, max_seqlen, hq, hkv, head_dim, block, topk, scale);
  if (st != MOBA_OK) return st;
  if (total <= 0 || max_seqlen > total) return MOBA_ERR_INVALID_ARG;
  if ((long long)total * hq >= (1ll << 31)) return MOBA_ERR_UNSUPPORTED;
  Shape s{nseq, max_seqlen, hq, hkv, head_dim, block, topk};
  s.cu = cu;
  s.total = total;
  *out = s;
  return MOBA_OK;
}

// backward workspace of a validated shape: all kv-heads at once, *min_bytes one per pass
size_t bwd_workspace(const Shape& s0, size_t* min_bytes) {
  // every causal block selected: the backward of dense causal attention
  const Shape s = all_blocks(s0) ? dense_shape(s0) : s0;
  if (!moba::bwd_supported(s)) return 0;
  const BwdLayout one = make_bwd_layout(s, 1);
  if (!bwd_layout_ok(one)) return 0;
  if (min_bytes) *min_bytes = one.total;
  for (int ng = s.hkv; ng >= 1; --ng) {
    const BwdLayout L = make_bwd_layout(s, ng);
    if (bwd_layout_ok(L)) return L.total;
  }
  return one.total;
}

// the whole backward for a validated shape (a uniform batch or packed sequences)
int run_backward(const Shape& s0, const void* q, const void* k, const void* v,
                 const void* out, const float* lse, const int32_t* idx, const void* dout,
                 float scale, void* dq, void* dk, void* dv, void* workspace,
                 size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !out || !lse || !idx || !dout || !dq || !dk || !dv || !workspace)
    return MOBA_ERR_INVALID_ARG;
  // every causal block selected (the only valid idx then): the backward of dense causal
  // attention, one block of the whole sequence with no history part
  const Shape s = all_blocks(s0) ? dense_shape(s0) : s0;
  if (((uintptr_t)workspace & (kAlign - 1)) != 0) return MOBA_ERR_INVALID_ARG;
  if (!moba::bwd_supported(s)) return MOBA_ERR_UNSUPPORTED;
  const int hkv = s.hkv;
  int ng = hkv;
  BwdLayout L = make_bwd_layout(s, ng);
  while (ng > 1 && (L.total > workspace_bytes || !bwd_layout_ok(L)))
    L = make_bwd_layout(s, --ng);
  if (L.total > workspace_bytes) return MOBA_ERR_WORKSPACE;
  if (!bwd_layout_ok(L)) return MOBA_ERR_UNSUPPORTED;

  char* ws = static_cast<char*>(workspace);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const uint16_t* qb = static_cast<const uint16_t*>(q);
  const uint16_t* kb = static_cast<const uint16_t*>(k);
  const uint16_t* vb = static_cast<const uint16_t*>(v);
  const uint16_t* gb = static_cast<const uint16_t*>(dout);
  float* delta = reinterpret_cast<float*>(ws + L.delta);
  float* dq_part = reinterpret_cast<float*>(ws + L.dq_part);
  MOBA_TRY(moba::launch_bwd_delta(s, static_cast<const uint16_t*>(out), gb, delta, hs));
  for (int g0 = 0; g0 < hkv; g0 += ng) {
    const int ngc = ng < hkv - g0 ? ng : hkv - g0;
    const int nlc = s.b * ngc * s.nb();
    const int32_t* list_offsets = nullptr;
    uint16_t* dense_rows = reinterpret_cast<uint16_t*>(ws + L.dense_rows);
    float* dense_meta = reinterpret_cast<float*>(ws + L.dense_meta);
    if (s.KH() > 0) {
      int32_t* lo = reinterpret_cast<int32_t*>(ws + L.list_offsets);
      int32_t* tile_offsets = reinterpret_cast<int32_t*>(ws + L.tile_offsets);
      int4* tiles = reinterpret_cast<int4*>(ws + L.tiles);
      uint32_t* ent = reinterpret_cast<uint32_t*>(ws + L.entries);
      MOBA_TRY(moba::launch_index(s, idx, g0, ngc, moba::bwd_tile_rows(),
                                  reinterpret_cast<int32_t*>(ws + L.chunk_counts),
                                  reinterpret_cast<int32_t*>(ws + L.list_count), lo,
                                  tile_offsets, tiles, ent, L.n_entries, hs));
      const BwdLayout Lc = make_bwd_layout(s, ngc);
      MOBA_TRY(moba::launch_bwd_dq_history(s, qb, kb, vb, gb, lse, delta, scale, g0, ngc,
                                           tiles, tile_offsets + nlc, (int)Lc.max_tiles,
                                           ent, dq_part, hs));
      MOBA_TRY(moba::launch_bwd_densify(s, qb, gb, lse, delta, g0, ngc, tiles,
                                        tile_offsets + nlc, (int)Lc.max_tiles, ent,
                                        dense_rows, dense_meta, hs));
      list_offsets = lo;
    }
    MOBA_TRY(moba::launch_bwd_dq_current(s, qb, kb, vb, gb, lse, delta, scale, g0, ngc,
                                         dq_part, static_cast<uint16_t*>(dq), hs));
    MOBA_TRY(moba::launch_bwd_dkdv(s, qb, kb, vb, gb, lse, delta, scale, g0, ngc,
                                   list_offsets, dense_rows, dense_meta,
                                   static_cast<uint16_t*>(dk), static_cast<uint16_t*>(dv),
                                   hs));
  }
  return MOBA_OK;
}

}  // namespace

extern "C" {

int moba_forward(const void* q, const void* k, const void* v, int batch, int seqlen,
                 int hq, int hkv, int head_dim, int block, int topk, float scale,
                 void* out, float* lse, int32_t* idx, void* workspace,
                 size_t workspace_bytes, void* stream) {
  return forward_impl(q, k, v, batch, seqlen, hq, hkv, head_dim, block, topk, scale, out,
                      lse, idx, workspace, workspace_bytes, stream, nullptr, nullptr);
}

int moba_dense_forward(const void* q, const void* k, const void* v, int batch, int seqlen,
                       int hq, int hkv, int head_dim, float scale, void* out, float* lse,
                       void* stream) {
  // one block of seqlen tokens (rounded up to whole 16-key subtiles; keys past seqlen
  // are never read) and topk 1: the current-block kernel alone is dense causal
  // attention, with no history part to merge
  const int blk = (seqlen + 15) / 16 * 16;
  const int st = check(batch, seqlen, hq, hkv, head_dim, blk > 0 ? blk : 16, 1, scale);
  if (st != MOBA_OK) return st;
  if (!q || !k || !v || !out || !lse) return MOBA_ERR_INVALID_ARG;
  const Shape s{batch, seqlen, hq, hkv, head_dim, blk, 1};
  if (moba::launch_attn_current(s, static_cast<const uint16_t*>(q),
                                static_cast<const uint16_t*>(k),
                                static_cast<const uint16_t*>(v), scale, 0, hkv, nullptr,
                                nullptr, static_cast<uint16_t*>(out), lse,
                                static_cast<hipStream_t>(stream)) != hipSuccess)
    return MOBA_ERR_HIP;
  return MOBA_OK;
}

// ------------------------------------------------------------------- decode
namespace {

int decode_check(int batch, int n_new, int kv_len, int hq, int hkv, int head_dim,
                 float scale) {
  if (batch <= 0 || n_new <= 0 || kv_len <= 0 || hq <= 0 || hkv <= 0 || head_dim <= 0)
    return MOBA_ERR_INVALID_ARG;
  if (hq % hkv != 0 || n_new > kv_len) return MOBA_ERR_INVALID_ARG;
  if (!isfinite(scale)) return MOBA_ERR_INVALID_ARG;
  if (scale <= 0.f) return MOBA_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return MOBA_ERR_UNSUPPORTED;
  if ((long long)(hq / hkv) * n_new > moba::decode_max_rows()) return MOBA_ERR_UNSUPPORTED;
  if (batch > 65535 || (long long)hkv * (((hq / hkv) * n_new + 31) / 32) > 65535)
    return MOBA_ERR_UNSUPPORTED;
  // 32-bit buffer offsets within a 32-key subtile, and int token counts
  if ((long long)32 * hkv * head_dim * 2 >= (1ll << 31)) return MOBA_ERR_UNSUPPORTED;
  if ((long long)batch * kv_len >= (1ll << 31)) return MOBA_ERR_UNSUPPORTED;
  return MOBA_OK;
}

}  // namespace

size_t moba_decode_workspace_bytes(int batch, int n_new, int kv_len, int hq, int hkv,
                                   int head_dim) {
  if (decode_check(batch, n_new, kv_len, hq, hkv, head_dim, 1.f) != MOBA_OK) return 0;
  const moba::DecodePlan p = moba::decode_plan(batch, n_new, kv_len, hq, hkv, head_dim);
  return align_up(p.part_o_bytes) + align_up(p.part_lse_bytes);
}

int moba_decode(const void* q, const void* k, const void* v, int batch, int n_new,
                int kv_len, int hq, int hkv, int head_dim, float scale, void* out,
                float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  const int st = decode_check(batch, n_new, kv_len, hq, hkv, head_dim, scale);
  if (st != MOBA_OK) return st;
  if (!q || !k || !v || !out || !lse || !workspace) return MOBA_ERR_INVALID_ARG;
  if (((uintptr_t)workspace & (kAlign - 1)) != 0) return MOBA_ERR_INVALID_ARG;
  const moba::DecodePlan p = moba::decode_plan(batch, n_new, kv_len, hq, hkv, head_dim);
  if (align_up(p.part_o_bytes) + align_up(p.part_lse_bytes) > workspace_bytes)
    return MOBA_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  float* part_o = reinterpret_cast<float*>(ws);
  float* part_lse = reinterpret_cast<float*>(ws + align_up(p.part_o_bytes));
  if (moba::launch_decode(batch, n_new, kv_len, hq, hkv, head_dim, scale, p,
                          static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                          static_cast<const uint16_t*>(v), part_o, part_lse,
                          static_cast<uint16_t*>(out), lse,
                          static_cast<hipStream_t>(stream)) != hipSuccess)
    return MOBA_ERR_HIP;
  return MOBA_OK;
}

int moba_forward_profile(const void* q, const void* k, const void* v, int batch,
                         int seqlen, int hq, int hkv, int head_dim, int block, int topk,
                         float scale, void* out, float* lse, int32_t* idx,
                         void* workspace, size_t workspace_bytes, void* stream,
                         float* stage_ms) {
  if (!stage_ms) return MOBA_ERR_INVALID_ARG;
  return forward_impl(q, k, v, batch, seqlen, hq, hkv, head_dim, block, topk, scale, out,
                      lse, idx, workspace, workspace_bytes, stream, stage_ms, nullptr);
}

int moba_forward_timed(const void* q, const void* k, const void* v, int batch, int seqlen,
                       int hq, int hkv, int head_dim, int block, int topk, float scale,
                       void* out, float* lse, int32_t* idx, void* workspace,
                       size_t workspace_bytes, void* stream, void* const* stage_events) {
  if (!stage_events) return MOBA_ERR_INVALID_ARG;
  for (int i = 0; i <= MOBA_NUM_STAGES; ++i)
    if (!stage_events[i]) return MOBA_ERR_INVALID_ARG;
  return forward_impl(q, k, v, batch, seqlen, hq, hkv, head_dim, block, topk, scale, out,
                      lse, idx, workspace, workspace_bytes, stream, nullptr, stage_events);
}

// ------------------------------------------------------------------- packed sequences
size_t moba_varlen_workspace_bytes(int nseq, int total, int max_seqlen, int hq, int hkv,
                                   int head_dim, int block, int topk, size_t* min_bytes) {
  if (min_bytes) *min_bytes = 0;
  Shape s{};
  static const int32_t kDummy = 0;   // only the null-ness of cu matters for sizing
  if (varlen_shape(nseq, total, max_seqlen, hq, hkv, head_dim, block, topk, 1.f, &kDummy,
                   &s) != MOBA_OK)
    return 0;
  if (all_blocks(s)) {          // dense causal: no workspace is used
    if (min_bytes) *min_bytes = kAlign;
    return kAlign;
  }
  const Layout one = make_layout(s, 1);
  if (!layout_ok(one)) return 0;
  if (min_bytes) *min_bytes = one.total;
  for (int ng = hkv; ng >= 1; --ng) {
    const Layout L = make_layout(s, ng);
    if (layout_ok(L)) return L.total;
  }
  return one.total;
}

int moba_forward_varlen(const void* q, const void* k, const void* v,
                        const int32_t* cu_seqlens, int nseq, int total, int max_seqlen,
                        int hq, int hkv, int head_dim, int block, int topk, float scale,
                        void* out, float* lse, int32_t* idx, void* workspace,
                        size_t workspace_bytes, void* stream) {
  if (!cu_seqlens) return MOBA_ERR_INVALID_ARG;
  Shape s{};
  const int st = varlen_shape(nseq, total, max_seqlen, hq, hkv, head_dim, block, topk, scale,
                              cu_seqlens, &s);
  if (st != MOBA_OK) return st;
  return run_forward(s, q, k, v, scale, out, lse, idx, workspace, workspace_bytes, stream,
                     nullptr, nullptr);
}

// ------------------------------------------------------------------- key convolution
int moba_key_short_conv(const void* k, const float* weight, const int32_t* cu_seqlens,
                        int batch, int seqlen, int total, int hkv, int head_dim, int block,
                        int width, void* out, void* stream) {
  Shape s{};
  int st;
  if (cu_seqlens) {
    st = varlen_shape(batch, total, seqlen, hkv, hkv, head_dim, block, 1, 1.f, cu_seqlens,
                      &s);
  } else {
    st = check(batch, seqlen, hkv, hkv, head_dim, block, 1, 1.f);
    s = Shape{batch, seqlen, hkv, hkv, head_dim, block, 1};
  }
  if (st != MOBA_OK) return st;
  if (width < 1) return MOBA_ERR_INVALID_ARG;
  if (width > moba::conv_max_width()) return MOBA_ERR_UNSUPPORTED;
  if (!k || !weight || !out) return MOBA_ERR_INVALID_ARG;
  return hip_status(moba::launch_key_conv(s, static_cast<const uint16_t*>(k), weight, width,
                                          static_cast<uint16_t*>(out),
                                          static_cast<hipStream_t>(stream)));
}

}  // extern "C"

// ------------------------------------------------------------------- stages
namespace {
// The index stage packs a slot into 5 or 6 bits: at most 64 history slots, and the
// limits of a sparse shape (which check() waives when every block is selected).
bool index_unsupported(int seqlen, int hq, int hkv, int block, int topk) {
  if (topk - 1 > moba::gate_max_history()) return true;
  if ((seqlen + block - 1) / block > kMaxBlocks) return true;
  return (long long)seqlen * (hq / hkv) >= (1ll << (32 - moba::entry_slot_bits(topk)));
}

// The history stage's tile list for kv_count kv-heads: tile rows, tile count bound,
// and the workspace (tile offsets, the tiles, and a second tile array for a permuted
// order).
struct HistoryTiles {
  int tile_m;
  long long nlists, max_tiles;
  size_t offsets_bytes, tiles_bytes;
};
HistoryTiles history_tiles(const Shape& s, int kv_count) {
  HistoryTiles h;
  const long long n_entries = (long long)s.b * kv_count * s.G() * entries_per_head(s);
  h.tile_m = moba::history_tile_rows(s, n_entries);
  h.nlists = (long long)s.b * kv_count * s.nb();
  h.max_tiles = (n_entries + h.tile_m - 1) / h.tile_m + h.nlists;
  h.offsets_bytes = align_up((size_t)(h.nlists + 2) * sizeof(int32_t));
  h.tiles_bytes = align_up((size_t)h.max_tiles * sizeof(int4));
  return h;
}
size_t history_stage_bytes(const Shape& s, int kv_count) {
  const HistoryTiles h = history_tiles(s, kv_count);
  return h.offsets_bytes + 2 * h.tiles_bytes;
}
}  // namespace

extern "C" {
size_t moba_stage_workspace_bytes(int batch, int seqlen, int hq, int hkv, int head_dim,
                                  int block, int topk) {
  if (check(batch, seqlen, hq, hkv, head_dim, block, topk, 1.f) != MOBA_OK) return 0;
  const Shape s{batch, seqlen, hq, hkv, head_dim, block, topk};
  const Layout L = make_layout(s, hkv);
  // pool partials, or hi/lo centroids, or the index scratch (chunk counts + counts +
  // tile offsets)
  const size_t a = L.cent;
  const size_t b2 = align_up((size_t)s.b * s.hkv * s.nb() * s.d * sizeof(uint16_t)) * 2;
  const size_t c = L.tiles - L.chunk_counts;
  size_t m = a > b2 ? a : b2;
  m = m > c ? m : c;
  const size_t h = s.KH() > 0 ? history_stage_bytes(s, s.hkv) : 0;
  return m > h ? m : h;
}

int moba_pool_centroids(const void* k, int batch, int seqlen, int hkv, int head_dim,
                        int block, float* centroids, void* workspace,
                        size_t workspace_bytes, void* stream) {
  int st = check(batch, seqlen, hkv, hkv, head_dim, block, 1, 1.f);
  if (st != MOBA_OK) return st;
  if (!k || !centroids || !workspace) return MOBA_ERR_INVALID_ARG;
  const Shape s{batch, seqlen, hkv, hkv, head_dim, block, 1};
  const Layout L = make_layout(s, 1);
  if (L.cent > workspace_bytes) return MOBA_ERR_WORKSPACE;
  return hip_status(moba::launch_pool(s, static_cast<const uint16_t*>(k),
                                      reinterpret_cast<float*>(workspace), centroids, nullptr,
                                      nullptr, static_cast<hipStream_t>(stream)));
}

int moba_gate_topk(const void* q, const float* centroids, int batch, int seqlen, int hq,
                   int hkv, int head_dim, int block, int topk, int32_t* idx,
                   void* workspace, size_t workspace_bytes, void* stream) {
  int st = check(batch, seqlen, hq, hkv, head_dim, block, topk, 1.f);
  if (st != MOBA_OK) return st;
  if (!q || !centroids || !idx || !workspace) return MOBA_ERR_INVALID_ARG;
  const Shape s{batch, seqlen, hq, hkv, head_dim, block, topk};
  if (all_blocks(s)) return hip_status(moba::launch_idx_all_blocks(s, idx,
                                                                   static_cast<hipStream_t>(stream)));
  const size_t n = (size_t)s.b * s.hkv * s.nb() * s.d;
  const size_t half = align_up(n * sizeof(uint16_t));
  if (2 * half > workspace_bytes) return MOBA_ERR_WORKSPACE;
  uint16_t* chi = static_cast<uint16_t*>(workspace);
  uint16_t* clo = reinterpret_cast<uint16_t*>(static_cast<char*>(workspace) + half);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  MOBA_TRY(moba::launch_centroid_split(s, centroids, chi, clo, hs));
  return hip_status(
      moba::launch_gate(s, static_cast<const uint16_t*>(q), chi, clo, idx, hs));
}

int64_t moba_index_entries(int batch, int seqlen, int hq, int hkv, int block, int topk,
                           int kv_count) {
  if (check(batch, seqlen, hq, hkv, 64, block, topk, 1.f) != MOBA_OK) return -1;
  if (index_unsupported(seqlen, hq, hkv, block, topk)) return -1;
  if (kv_count <= 0 || kv_count > hkv) return -1;
  const Shape s{batch, seqlen, hq, hkv, 64, block, topk};
  return (int64_t)s.b * kv_count * s.G() * entries_per_head(s);
}

int moba_build_index(const int32_t* idx, int batch, int seqlen, int hq, int hkv,
                     int block, int topk, int kv_begin, int kv_count,
                     int32_t* list_offsets, uint32_t* entries, void* workspace,
                     size_t workspace_bytes, void* stream) {
  int st = check(batch, seqlen, hq, hkv, 64, block, topk, 1.f);
  if (st != MOBA_OK) return st;
  if (!idx || !list_offsets || !entries || !workspace) return MOBA_ERR_INVALID_ARG;
  if (kv_begin < 0 || kv_count <= 0 || kv_begin + kv_count > hkv) return MOBA_ERR_INVALID_ARG;
  if (topk < 2) return MOBA_ERR_UNSUPPORTED;  // no history slots, no index
  if (index_unsupported(seqlen, hq, hkv, block, topk)) return MOBA_ERR_UNSUPPORTED;
  const Shape s{batch, seqlen, hq, hkv, 64, block, topk};
  const size_t nlists = (size_t)s.b * kv_count * s.nb();
  const size_t cc = align_up((size_t)s.b * kv_count * moba::index_chunks(s) * s.nb() *
                             sizeof(int32_t));
  const size_t lc = align_up(nlists * sizeof(int32_t));
  const size_t to = align_up((nlists + 2) * sizeof(int32_t));
  if (cc + lc + to > workspace_bytes) return MOBA_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  return hip_status(moba::launch_index(
      s, idx, kv_begin, kv_count, moba::history_tile_rows(),
      reinterpret_cast<int32_t*>(ws), reinterpret_cast<int32_t*>(ws + cc), list_offsets,
      reinterpret_cast<int32_t*>(ws + cc + lc), nullptr, entries,
      (long long)s.b * kv_count * s.G() * entries_per_head(s),
      static_cast<hipStream_t>(stream)));
}

int moba_history_partials(const void* q, const void* k, const void* v, int batch,
                          int seqlen, int hq, int hkv, int head_dim, int block, int topk,
                          float scale, int kv_begin, int kv_count,
                          const int32_t* list_offsets, const uint32_t* entries,
                          uint32_t tile_order_seed, void* part_o, float* part_lse,
                          void* workspace, size_t workspace_bytes, void* stream) {
  int st = check(batch, seqlen, hq, hkv, head_dim, block, topk, scale);
  if (st != MOBA_OK) return st;
  if (!q || !k || !v || !list_offsets || !entries || !part_o || !part_lse || !workspace)
    return MOBA_ERR_INVALID_ARG;
  if (kv_begin < 0 || kv_count <= 0 || kv_begin + kv_count > hkv) return MOBA_ERR_INVALID_ARG;
  if (topk < 2) return MOBA_ERR_UNSUPPORTED;  // no history slots
  if (index_unsupported(seqlen, hq, hkv, block, topk)) return MOBA_ERR_UNSUPPORTED;
  const Shape s{batch, seqlen, hq, hkv, head_dim, block, topk};
  const HistoryTiles h = history_tiles(s, kv_count);
  if (h.max_tiles >= (1ll << 31)) return MOBA_ERR_UNSUPPORTED;
  if (h.offsets_bytes + 2 * h.tiles_bytes > workspace_bytes) return MOBA_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  int32_t* tile_offsets = reinterpret_cast<int32_t*>(ws);
  int4* tiles = reinterpret_cast<int4*>(ws + h.offsets_bytes);
  int4* tmp = reinterpret_cast<int4*>(ws + h.offsets_bytes + h.tiles_bytes);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  MOBA_TRY(moba::launch_tiles(list_offsets, (int)h.nlists, h.tile_m, (int)h.max_tiles,
                              tile_offsets, tiles, tile_order_seed, tmp, hs));
  return hip_status(moba::launch_attn_history(
      s, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
      static_cast<const uint16_t*>(v), scale, kv_begin, kv_count, tiles,
      tile_offsets + h.nlists, (int)h.max_tiles, entries, static_cast<uint16_t*>(part_o),
      part_lse, hs));
}

int moba_current_merge(const void* q, const void* k, const void* v, int batch, int seqlen,
                       int hq, int hkv, int head_dim, int block, int topk, float scale,
                       int kv_begin, int kv_count, const void* part_o,
                       const float* part_lse, void* out, float* lse, void* stream) {
  int st = check(batch, seqlen, hq, hkv, head_dim, block, topk, scale);
  if (st != MOBA_OK) return st;
  if (!q || !k || !v || !out || !lse) return MOBA_ERR_INVALID_ARG;
  if (topk > 1 && (!part_o || !part_lse)) return MOBA_ERR_INVALID_ARG;
  if (kv_begin < 0 || kv_count <= 0 || kv_begin + kv_count > hkv) return MOBA_ERR_INVALID_ARG;
  const Shape s{batch, seqlen, hq, hkv, head_dim, block, topk};
  return hip_status(moba::launch_attn_current(
      s, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
      static_cast<const uint16_t*>(v), scale, kv_begin, kv_count,
      static_cast<const uint16_t*>(part_o), part_lse, static_cast<uint16_t*>(out), lse,
      static_cast<hipStream_t>(stream)));
}

// ------------------------------------------------------------------- backward
size_t moba_backward_workspace_bytes(int batch, int seqlen, int hq, int hkv,
                                     int head_dim, int block, int topk,
                                     size_t* min_bytes) {
  if (min_bytes) *min_bytes = 0;
  if (check(batch, seqlen, hq, hkv, head_dim, block, topk, 1.f) != MOBA_OK) return 0;
  return bwd_workspace(Shape{batch, seqlen, hq, hkv, head_dim, block, topk}, min_bytes);
}

int moba_backward(const void* q, const void* k, const void* v, const void* out,
                  const float* lse, const int32_t* idx, const void* dout, int batch,
                  int seqlen, int hq, int hkv, int head_dim, int block, int topk,
                  float scale, void* dq, void* dk, void* dv, void* workspace,
                  size_t workspace_bytes, void* stream) {
  const int st = check(batch, seqlen, hq, hkv, head_dim, block, topk, scale);
  if (st != MOBA_OK) return st;
  return run_backward(Shape{batch, seqlen, hq, hkv, head_dim, block, topk}, q, k, v, out,
                      lse, idx, dout, scale, dq, dk, dv, workspace, workspace_bytes, stream);
}

size_t moba_backward_varlen_workspace_bytes(int nseq, int total, int max_seqlen, int hq,
                                            int hkv, int head_dim, int block, int topk,
                                            size_t* min_bytes) {
  if (min_bytes) *min_bytes = 0;
  Shape s{};
  static const int32_t kDummy = 0;   // only the null-ness of cu matters for sizing
  if (varlen_shape(nseq, total, max_seqlen, hq, hkv, head_dim, block, topk, 1.f, &kDummy,
                   &s) != MOBA_OK)
    return 0;
  return bwd_workspace(s, min_bytes);
}

int moba_backward_varlen(const void* q, const void* k, const void* v, const void* out,
                         const float* lse, const int32_t* idx, const void* dout,
                         const int32_t* cu_seqlens, int nseq, int total, int max_seqlen,
                         int hq, int hkv, int head_dim, int block, int topk, float scale,
                         void* dq, void* dk, void* dv, void* workspace,
                         size_t workspace_bytes, void* stream) {
  if (!cu_seqlens) return MOBA_ERR_INVALID_ARG;
  Shape s{};
  const int st = varlen_shape(nseq, total, max_seqlen, hq, hkv, head_dim, block, topk, scale,
                              cu_seqlens, &s);
  if (st != MOBA_OK) return st;
  return run_backward(s, q, k, v, out, lse, idx, dout, scale, dq, dk, dv, workspace,
                      workspace_bytes, stream);
}

}  // extern "C"

// ------------------------------------------------------------------- no-allocation forward
// moba_forward for callers that cannot allocate: the workspace is a fixed device array of
// the library, one copy per GPU, which lives until the process ends.  Host code never
// passes the array's name to a kernel or a HIP call (it stands for a host-side shadow,
// not for device memory): the device address comes from hipGetSymbolAddress, taken once
// per device with that device current, and only that address is used afterwards.
static constexpr size_t kScratchBytes = (size_t)128 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// the scratch address on the current device, looked up on the first call there
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MOBA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MOBA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return MOBA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOBA_OK;
}

}  // namespace

extern "C" {

int moba_forward_noalloc(const void* q, const void* k, const void* v, int batch, int seqlen,
                         int hq, int hkv, int head_dim, int block, int topk, float scale,
                         void* out, float* lse, int32_t* idx, void* stream) {
  const int st = check(batch, seqlen, hq, hkv, head_dim, block, topk, scale);
  if (st != MOBA_OK) return st;
  if (!q || !k || !v || !out || !lse || !idx) return MOBA_ERR_INVALID_ARG;
  // the one-kv-head-per-pass size must fit the scratch; this is decided on the host
  // before any device work, like every other check
  const Shape s{batch, seqlen, hq, hkv, head_dim, block, topk};
  if (!all_blocks(s)) {
    const Layout one = make_layout(s, 1);
    if (!layout_ok(one)) return MOBA_ERR_UNSUPPORTED;
    if (one.total > kScratchBytes) return MOBA_ERR_WORKSPACE;
  }
  void* ws = nullptr;
  const int sa = scratch_address(&ws);
  if (sa != MOBA_OK) return sa;
  return run_forward(s, q, k, v, scale, out, lse, idx, ws, kScratchBytes, stream, nullptr,
                     nullptr);
}

}  // extern "C"
