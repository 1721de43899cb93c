// cp_api.hip -- the extern "C" entry points of libcp (declared in cp.h).
//
// Host code only: argument validation (everything a host can check is
// checked before anything is enqueued), the attention plan (kernel choice,
// query tiling, key splits), and the launches.  No allocation, no global
// mutable state, no stream synchronisation.
#include <atomic>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "attn_common.h"

// Key-split partials of cp_attn_chunk_with_past_noalloc.  Host code never uses this
// name as a device address (in host code it is only a stand-in for the symbol): the
// address comes from hipGetSymbolAddress, once per device (scratch_on_current_device).
static __device__ __align__(256) unsigned char scratch[CP_ATTN_SCRATCH_BYTES];

namespace cp {
int mfma_keys_per_tile(int D, bool explicit_tiling, int small_rows);
int mfma_rows_per_tile(int D, bool explicit_tiling, int small_rows);
int mfma_wgs_per_cu(int D, bool explicit_tiling, int small_rows);
int valu_keys(int D);

namespace {

constexpr int kAbiVersion = 4;
constexpr int kNumCU = 256;
// Fewest key tiles per piece of a balanced split (each workgroup pays a prologue and the
// first tile's latency, about two tiles' time).
constexpr int kPlanMinTiles = 4;

int to_status(hipError_t e) { return e == hipSuccess ? CP_OK : CP_ERR_HIP; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t esize(int dtype) { return dtype == CP_BF16 ? 2 : 4; }

int check_cache(const cp_cache *c) {
  if (!c || !c->k || !c->v || !c->seen) return CP_ERR_ARG;
  if (c->dtype != CP_F32 && c->dtype != CP_BF16) return CP_ERR_DTYPE;
  if (c->reserved != 0 || (c->ring != 0 && c->ring != 1)) return CP_ERR_ARG;
  if (c->B < 0 || c->nKV < 1 || c->cap < 1 || c->D < 1) return CP_ERR_SHAPE;
  if (c->sink < 0 || c->sink >= c->cap) return CP_ERR_ARG;
  return CP_OK;
}

size_t round256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Device address of `scratch` on each device, resolved on the first call that needs it
// with that device current (each GPU holds its own copy of the array).
constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

int scratch_on_current_device(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return CP_ERR_HIP;
  void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return CP_ERR_HIP;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return CP_OK;
}

}  // namespace

AttnPlan plan_attention(const cp_cache &c, const cp_attn_args &a, bool for_workspace) {
  AttnPlan pl{};
  const int G = a.H / c.nKV;
  const bool aligned = aligned16(a.q) && aligned16(a.k_new) && aligned16(a.v_new) &&
                       aligned16(a.out) && aligned16(c.k) && aligned16(c.v) &&
                       (!a.q_cos || (aligned16(a.q_cos) && aligned16(a.q_sin)));
  const bool ext = a.mask != nullptr || (a.flags & CP_ATTN_FULL_TILES);
  const bool mfma_d = c.D == 64 || c.D == 128 || c.D == 256;
  // all rows of one KV head fit 64: the small-rows configuration
  pl.small_rows = static_cast<long>(a.C) * G <= 64 ? 1 : 0;
  // medium rows (D = 128, in-kernel rule): the rows of one KV head fit 128
  if (!pl.small_rows && c.D == 128 && !ext && static_cast<long>(a.C) * G <= 128)
    pl.small_rows = 3;
  const int rows = mfma_d ? mfma_rows_per_tile(c.D, ext, pl.small_rows) : 0;
  pl.mfma = c.dtype == CP_BF16 && mfma_d && G <= rows && !(a.flags & CP_ATTN_FORCE_GENERIC) &&
            aligned;
  int hgroups = 1;
  if (pl.mfma) {
    pl.rows = rows;
    pl.qpos = rows / G;
    pl.kt = mfma_keys_per_tile(c.D, ext, pl.small_rows);
  } else {
    const int hb = G < 16 ? G : 16;
    hgroups = (G + hb - 1) / hb;
    pl.qpos = 16 / hb;
    pl.kt = valu_keys(c.D);
  }
  pl.qtiles = (a.C + pl.qpos - 1) / pl.qpos;
  pl.splits = 1;
  const long base = static_cast<long>(pl.qtiles) * hgroups * c.B * c.nKV;
  // keys one query tile can see: the live past (at most the capacity, or the caller's
  // bound on seen) and the chunk, or the window's reach
  long keys = static_cast<long>(a.max_seen > 0 && a.max_seen < c.cap ? a.max_seen : c.cap) + a.C;
  if (a.window > 0 && !a.mask) {
    const long wk = static_cast<long>(a.window) + pl.qpos + c.sink;
    if (wk < keys) keys = wk;
  }
  const long tiles = (keys + pl.kt - 1) / pl.kt;
  const int forced = static_cast<int>((a.flags >> 8) & 0xffu);
  // Few query tiles: split the keys so that more CUs work -- each split writes
  // partials that a second kernel merges.  The matrix-core kernel keeps >= 2 key tiles
  // per split (its prologue and first-tile latency is paid per workgroup; with the
  // merge reading all splits in one round, 2 measured best: the 864-key D = 256 chunk
  // step 18.75 -> 18.50 us, the 640-key ring step 22.05 -> 20.59 us against 3); the
  // vector-ALU kernel's 16-key tiles each cost a memory round trip that their
  // arithmetic does not hide, so it goes down to one tile per split.  The tile count is
  // a bound (from the capacity or max_seen; the live length is on the device), so a
  // split can get one tile less than this.  Rounded up: an odd count leaves one split a
  // single tile rather than one split three (the 864-key chunk: 14 splits 13.96 us per
  // call, 13 or 12 splits 15.4).
  const long per = pl.mfma ? 2 : 1;
  // as many splits as fill the CUs once (rounded down: a partial second round of
  // workgroups would double the time of the last ones)
  auto split_for = [&](long wg_per_cu) {
    long s = wg_per_cu * kNumCU / base;
    if (s > (tiles + per - 1) / per) s = (tiles + per - 1) / per;
    if (s > 64) s = 64;
    return s > 1 ? static_cast<int>(s) : 1;
  };
  const bool split_ok = !(a.flags & CP_ATTN_NO_SPLIT) && base > 0 && base < kNumCU;
  if (forced > 0) {
    pl.splits = forced > 64 ? 64 : forced;
  } else if (split_ok) {
    pl.splits = split_for(pl.mfma ? mfma_wgs_per_cu(c.D, ext, pl.small_rows) : 2);
  }
  // Small rows whose splits each stream many tiles (long decode contexts): the deep-ring
  // configuration, three workgroups per CU (in-kernel rule only).
  if (pl.mfma && pl.small_rows == 1 && !ext && tiles / pl.splits >= 24) {
    pl.small_rows = 2;
    if (forced == 0 && split_ok) pl.splits = split_for(mfma_wgs_per_cu(c.D, ext, 2));
  }
  // Balanced splits (standard matrix-core configuration): a device-side plan cuts each
  // sequence's keys by its own length.  The launch holds every item the plan can make:
  // with pieces of at least total / slots tiles there are at most slots + base of them
  // (plus the padding of the last group of 8 units).
  if ((a.flags & CP_ATTN_BALANCE) && pl.mfma && pl.small_rows == 0 && forced == 0 &&
      c.B <= kPlanMaxB && base > 0) {
    pl.planned = true;
    pl.splits = 1;
    pl.plan_slots = mfma_wgs_per_cu(c.D, ext, 0) * kNumCU;
    const long per = 8L * pl.qtiles;
    long grid = pl.plan_slots + base + per;
    grid = (grid + per - 1) / per * per;
    pl.plan_grid = static_cast<int>(grid);
  }
  const bool needs_ws = pl.splits > 1 || pl.planned;
  if (needs_ws && !for_workspace &&
      (!a.workspace || a.workspace_bytes < attn_workspace_bytes(c, a, pl))) {
    pl.splits = 1;
    pl.planned = false;
  }
  // XCD placement (blocks are dealt round-robin over the 8 XCDs, each with its own
  // L2).  A split call whose (split, sequence, KV head) groups are not a multiple of 8
  // pads their count to one, so that the query tiles of a group share an XCD and its
  // K/V is fetched once -- unless its query tiles are themselves a multiple of 8, where
  // the tile-minor order keeps every split of a tile on one XCD (with its queries).  The
  // merge deals whole units to the XCDs: the query tile when each tile's splits ran on
  // one XCD, else one 32-row group, so that the output lines of a unit are written
  // whole from one L2 (spread over the XCDs, two L2s write halves of a line).
  if (pl.mfma && !pl.planned && pl.splits > 1) {
    const long groups = static_cast<long>(pl.splits) * c.B * c.nKV;
    const bool tile_local = groups % 8 != 0 && pl.qtiles % 8 == 0;
    pl.xpad = groups % 8 != 0 && !tile_local && groups >= 8 ? 1 : 0;
    pl.xmerge = tile_local ? pl.rows / 32 : 1;
  }
  return pl;
}

// Rows of the split partials: the chunk rows, or for the matrix-core kernel every row
// of every query tile (fragment order, which includes the last tile's rows past C and,
// when G does not divide a tile's rows, its spare rows).
static size_t partial_rows(const cp_cache &c, const cp_attn_args &a, const AttnPlan &p) {
  if (p.mfma) return static_cast<size_t>(c.B) * c.nKV * p.qtiles * p.rows;
  return static_cast<size_t>(c.B) * a.H * a.C;
}

// Bytes per partial O element: the matrix-core kernel stores normalized bf16, the
// vector-ALU kernel fp32 sums.
static size_t partial_esize(const AttnPlan &p) { return p.mfma ? 2 : 4; }

// Planned mode: the plan (header, items, split entries), then the partials of at most
// plan_grid slots in fragment order, then their (m, l).
static size_t plan_bytes(const AttnPlan &p) {
  return round256(sizeof(int32_t) *
                  (kPlanHeaderInts + 2 * static_cast<size_t>(p.plan_grid) * kPlanItemInts));
}

size_t attn_workspace_bytes(const cp_cache &c, const cp_attn_args &a, const AttnPlan &p) {
  if (p.planned) {
    const size_t rows = static_cast<size_t>(p.plan_grid) * p.rows;
    return plan_bytes(p) + round256(rows * c.D * partial_esize(p)) +
           round256(rows * 2 * sizeof(float));
  }
  if (p.splits <= 1) return 0;
  const size_t rows = partial_rows(c, a, p);
  return round256(static_cast<size_t>(p.splits) * rows * c.D * partial_esize(p)) +
         round256(static_cast<size_t>(p.splits) * rows * 2 * sizeof(float));
}

hipError_t launch_attention(const cp_cache &c, const cp_attn_args &a, hipStream_t s) {
  const AttnPlan pl = plan_attention(c, a, false);
  AttnParams p{};
  p.q = a.q;
  p.kn = a.k_new;
  p.vn = a.v_new;
  p.kc = c.k;
  p.vc = c.v;
  p.out = a.out;
  p.sel = a.select_out;
  p.seen = c.seen;
  p.n_valid = a.n_valid;
  p.status = c.status;
  p.mask = a.mask;
  p.mld = a.mask_ld;
  p.mhs = a.mask_head_stride;
  p.mbs = a.mask_batch_stride;
  p.B = c.B;
  p.H = a.H;
  p.nKV = c.nKV;
  p.C = a.C;
  p.cap = c.cap;
  p.ring = c.ring;
  p.sink = c.sink;
  p.window = a.mask ? 0 : a.window;
  p.G = a.H / c.nKV;
  p.qpos = pl.qpos;
  p.qtiles = pl.qtiles;
  p.splits = pl.splits;
  p.full_tiles = (a.flags & CP_ATTN_FULL_TILES) ? 1 : 0;
  p.sl2e = a.scale * kLog2e;
  p.small_rows = pl.small_rows;
  p.cache = c;
  p.q_cos = a.q_cos;
  p.q_sin = a.q_sin;
  p.q_tables = a.q_tables;
  const bool advance = (a.flags & CP_ATTN_ADVANCE_SEEN) != 0;
  p.advance = advance && pl.splits > 1 ? 1 : 0;
  p.frag_rows = pl.mfma ? pl.rows : 0;
  p.xpad = static_cast<int16_t>(pl.xpad);
  p.xmerge = static_cast<int16_t>(pl.xmerge);
  if (pl.planned) {
    unsigned char *w = static_cast<unsigned char *>(a.workspace);
    const size_t rows = static_cast<size_t>(pl.plan_grid) * pl.rows;
    p.plan = reinterpret_cast<const int32_t *>(w);
    p.plan_grid = pl.plan_grid;
    p.plan_slots = pl.plan_slots;
    p.plan_kt = pl.kt;
    p.plan_tmin = kPlanMinTiles;
    p.wo = reinterpret_cast<float *>(w + plan_bytes(pl));
    p.wml = reinterpret_cast<float *>(w + plan_bytes(pl) +
                                      round256(rows * c.D * partial_esize(pl)));
    p.advance = advance ? 1 : 0;
  } else if (pl.splits > 1) {
    const size_t rows = partial_rows(c, a, pl);
    unsigned char *w = static_cast<unsigned char *>(a.workspace);
    p.wo = reinterpret_cast<float *>(w);
    p.wml = reinterpret_cast<float *>(
        w + round256(static_cast<size_t>(pl.splits) * rows * c.D * partial_esize(pl)));
  }
  if (static_cast<size_t>(c.B) * a.H * a.C == 0)
    return advance ? launch_advance_seen(c, a.C, a.n_valid, s) : hipSuccess;
  hipError_t e;
  if (pl.planned) {
    p.hb = p.G;
    p.hgroups = 1;
    e = launch_attn_plan(p, s);
    if (e == hipSuccess) e = launch_attn_mfma(p, c.D, s);
    if (e == hipSuccess) e = launch_attn_merge_plan(p, c.D, s);  // also advances seen
    return e;
  }
  if (pl.mfma) {
    p.hb = p.G;
    p.hgroups = 1;
    e = launch_attn_mfma(p, c.D, s);
  } else {
    p.hb = p.G < 16 ? p.G : 16;
    p.hgroups = (p.G + p.hb - 1) / p.hb;
    e = launch_attn_valu(p, c.D, c.dtype, s);
  }
  if (e != hipSuccess) return e;
  if (pl.splits == 1) return advance ? launch_advance_seen(c, a.C, a.n_valid, s) : e;
  return launch_attn_combine(p, c.D, c.dtype, s);  // also advances seen when asked
}

}  // namespace cp

using namespace cp;

extern "C" {

const char *cp_status_str(int status) {
  switch (status) {
    case CP_OK:
      return "ok";
    case CP_ERR_ARG:
      return "invalid argument (null pointer or out-of-range scalar)";
    case CP_ERR_SHAPE:
      return "unsupported or inconsistent shape";
    case CP_ERR_DTYPE:
      return "unsupported dtype";
    case CP_ERR_WINDOW:
      return "ring window too small for a padded append (cap <= C + sink)";
    case CP_ERR_STATE:
      return "rollback without a matching armed snapshot";
    case CP_ERR_WORKSPACE:
      return "workspace or snapshot buffer too small";
    case CP_ERR_HIP:
      return "HIP runtime error";
    case CP_ERR_SCRATCH:
      return "the call's key splits need more than the library's fixed scratch array "
             "(CP_ATTN_SCRATCH_BYTES); use cp_attn_chunk_with_past with a workspace";
    default:
      return "unknown status";
  }
}

int cp_abi_version(void) { return kAbiVersion; }

size_t cp_struct_size(int which) {
  switch (which) {
    case 0:
      return sizeof(cp_cache);
    case 1:
      return sizeof(cp_snapshot);
    case 2:
      return sizeof(cp_attn_args);
    default:
      return 0;
  }
}

int cp_rope_chunk(const void *x, void *y, const float *cos, const float *sin, int B, int Hx,
                  int C, int D, int Bt, int dtype, cp_stream_t stream) {
  if (dtype != CP_F32 && dtype != CP_BF16) return CP_ERR_DTYPE;
  if (B < 0 || Hx < 0 || C < 0 || D < 1) return CP_ERR_ARG;
  if (D % 2 != 0) return CP_ERR_SHAPE;
  if (Bt != 1 && Bt != B) return CP_ERR_ARG;
  if (static_cast<size_t>(B) * Hx * C == 0) return CP_OK;  // empty: pointers may be NULL
  if (!x || !y || !cos || !sin) return CP_ERR_ARG;
  return to_status(launch_rope(x, y, cos, sin, B, Hx, C, D, Bt, dtype,
                               static_cast<hipStream_t>(stream)));
}

int cp_rope_qk_chunk(const void *q, void *q_out, const void *k, void *k_out, const float *cos,
                     const float *sin, int B, int H, int nKV, int C, int D, int Bt, int dtype,
                     cp_stream_t stream) {
  if (dtype != CP_F32 && dtype != CP_BF16) return CP_ERR_DTYPE;
  if (B < 0 || H < 0 || nKV < 0 || C < 0 || D < 1) return CP_ERR_ARG;
  if (D % 2 != 0) return CP_ERR_SHAPE;
  if (Bt != 1 && Bt != B) return CP_ERR_ARG;
  const bool has_q = static_cast<size_t>(B) * H * C > 0;
  const bool has_k = static_cast<size_t>(B) * nKV * C > 0;
  if (!has_q && !has_k) return CP_OK;  // empty: pointers may be NULL
  if (!cos || !sin || (has_q && (!q || !q_out)) || (has_k && (!k || !k_out))) return CP_ERR_ARG;
  if (!has_q)
    return to_status(launch_rope(k, k_out, cos, sin, B, nKV, C, D, Bt, dtype,
                                 static_cast<hipStream_t>(stream)));
  return to_status(launch_rope2(q, q_out, H, k, k_out, has_k ? nKV : 0, cos, sin, B, C, D, Bt,
                                dtype, static_cast<hipStream_t>(stream)));
}

int cp_rope_qk_append_chunk(const cp_cache *cache, const void *q, void *q_out, const void *k,
                            void *k_out, const void *v, const float *cos, const float *sin, int H,
                            int C, int Bt, const int32_t *n_valid, cp_stream_t stream) {
  int st = check_cache(cache);
  if (st != CP_OK) return st;
  if (cache->ring) return CP_ERR_ARG;  // a ring append may evict rows the attention reads
  if (H < 0 || C < 0) return CP_ERR_ARG;
  if (cache->D % 2 != 0 || C > cache->cap) return CP_ERR_SHAPE;
  if (Bt != 1 && Bt != cache->B) return CP_ERR_ARG;
  if (static_cast<size_t>(cache->B) * C == 0) return CP_OK;  // empty: pointers may be NULL
  if (!k || !k_out || !v || !cos || !sin || (H > 0 && (!q || !q_out))) return CP_ERR_ARG;
  return to_status(launch_rope_qk_append(*cache, q, q_out, H, k, k_out, v, cos, sin, C, Bt,
                                         n_valid, static_cast<hipStream_t>(stream)));
}

int cp_rope_qk_snapshot_chunk(const cp_cache *cache, const void *q, void *q_out, const void *k,
                              void *k_out, const float *cos, const float *sin, int H, int C,
                              int Bt, const int32_t *n_valid, cp_snapshot *snap,
                              cp_stream_t stream) {
  int st = check_cache(cache);
  if (st != CP_OK) return st;
  if (!snap || !snap->buf || H < 0 || C < 0) return CP_ERR_ARG;
  if (cache->D % 2 != 0) return CP_ERR_SHAPE;
  if (cache->ring && cache->cap <= C + cache->sink) return CP_ERR_WINDOW;
  if (!cache->ring && C > cache->cap) return CP_ERR_SHAPE;
  if (Bt != 1 && Bt != cache->B) return CP_ERR_ARG;
  if (snap->bytes < cp_snapshot_bytes(cache, C)) return CP_ERR_WORKSPACE;
  const bool rows = static_cast<size_t>(cache->B) * C > 0;
  if (rows && (!k || !k_out || !cos || !sin || (H > 0 && (!q || !q_out)))) return CP_ERR_ARG;
  if (cache->B > 0) {
    st = to_status(launch_rope_qk_snapshot(*cache, q, q_out, H, k, k_out, cos, sin, C, Bt,
                                           n_valid, snap->buf, static_cast<hipStream_t>(stream)));
    if (st != CP_OK) return st;
  }
  snap->cache_k = cache->k;
  snap->C = C;
  snap->armed = 1;
  return CP_OK;
}

int cp_kv_append_rollback(const cp_cache *cache, const void *k_new, const void *v_new, int C,
                          cp_snapshot *snap, cp_stream_t stream) {
  int st = check_cache(cache);
  if (st != CP_OK) return st;
  if (!snap || !snap->buf || C < 0) return CP_ERR_ARG;
  if (!snap->armed || snap->cache_k != cache->k || snap->C != C) return CP_ERR_STATE;
  if (snap->bytes < cp_snapshot_bytes(cache, C)) return CP_ERR_STATE;
  if (static_cast<size_t>(cache->B) * C > 0 && (!k_new || !v_new)) return CP_ERR_ARG;
  st = to_status(launch_append_rollback(*cache, k_new, v_new, C, snap->buf,
                                        static_cast<hipStream_t>(stream)));
  if (st != CP_OK) return st;
  snap->armed = 0;
  return CP_OK;
}

int cp_kv_advance(const cp_cache *cache, int C, const int32_t *n_rows, cp_stream_t stream) {
  int st = check_cache(cache);
  if (st != CP_OK) return st;
  if (C < 0) return CP_ERR_ARG;
  if (!cache->ring && C > cache->cap) return CP_ERR_SHAPE;
  if (C == 0 || cache->B == 0) return CP_OK;
  return to_status(launch_advance_seen(*cache, C, n_rows, static_cast<hipStream_t>(stream)));
}

int cp_kv_append(const cp_cache *cache, const void *k_new, const void *v_new, int C,
                 const int32_t *n_rows, cp_stream_t stream) {
  int st = check_cache(cache);
  if (st != CP_OK) return st;
  if (C < 0) return CP_ERR_ARG;
  if (!cache->ring && C > cache->cap) return CP_ERR_SHAPE;
  if (C == 0 || cache->B == 0) return CP_OK;  // nothing appended; pointers may be NULL
  if (!k_new || !v_new) return CP_ERR_ARG;
  return to_status(
      launch_kv_append(*cache, k_new, v_new, C, n_rows, static_cast<hipStream_t>(stream)));
}

size_t cp_snapshot_bytes(const cp_cache *cache, int C) {
  if (check_cache(cache) != CP_OK || C < 0) return 0;
  return snapshot_header_bytes(cache->B) +
         2 * round256(static_cast<size_t>(cache->B) * cache->nKV * C * cache->D *
                      esize(cache->dtype));
}

int cp_kv_snapshot_padded_append(const cp_cache *cache, int C, const int32_t *n_valid,
                                 cp_snapshot *snap, cp_stream_t stream) {
  int st = check_cache(cache);
  if (st != CP_OK) return st;
  if (!snap || !snap->buf || C < 0) return CP_ERR_ARG;
  if (cache->ring && cache->cap <= C + cache->sink) return CP_ERR_WINDOW;
  if (!cache->ring && C > cache->cap) return CP_ERR_SHAPE;
  if (snap->bytes < cp_snapshot_bytes(cache, C)) return CP_ERR_WORKSPACE;
  st = to_status(launch_snapshot(*cache, C, n_valid, snap->buf, static_cast<hipStream_t>(stream)));
  if (st != CP_OK) return st;
  snap->cache_k = cache->k;
  snap->C = C;
  snap->armed = 1;
  return CP_OK;
}

int cp_kv_rollback_padded_append(const cp_cache *cache, cp_snapshot *snap, cp_stream_t stream) {
  int st = check_cache(cache);
  if (st != CP_OK) return st;
  if (!snap || !snap->buf) return CP_ERR_ARG;
  if (!snap->armed || snap->cache_k != cache->k || snap->C < 0) return CP_ERR_STATE;
  if (snap->bytes < cp_snapshot_bytes(cache, snap->C)) return CP_ERR_STATE;
  st = to_status(launch_rollback(*cache, snap->C, snap->buf, static_cast<hipStream_t>(stream)));
  if (st != CP_OK) return st;
  snap->armed = 0;
  return CP_OK;
}

static int check_attn(const cp_cache *cache, const cp_attn_args *a) {
  int st = check_cache(cache);
  if (st != CP_OK) return st;
  if (!a) return CP_ERR_ARG;
  const bool empty = static_cast<size_t>(cache->B) * a->C == 0;
  if (!empty && (!a->q || !a->k_new || !a->v_new || !a->out)) return CP_ERR_ARG;
  if (a->reserved != 0 || a->C < 0 || a->window < 0 || !std::isfinite(a->scale) || a->scale <= 0.f)
    return CP_ERR_ARG;
  if (a->H < 1 || a->H % cache->nKV != 0) return CP_ERR_SHAPE;
  if (cache->D > 256) return CP_ERR_SHAPE;
  if (!cache->ring && a->C > cache->cap) return CP_ERR_SHAPE;
  if (a->mask && (a->mask_ld < a->C || a->mask_head_stride < 0 || a->mask_batch_stride < 0))
    return CP_ERR_ARG;
  if (a->max_seen < 0 || (!a->q_cos) != (!a->q_sin)) return CP_ERR_ARG;
  if (a->q_cos) {
    if (a->q_tables != 1 && a->q_tables != cache->B) return CP_ERR_ARG;
    if (cache->D % 2 != 0) return CP_ERR_SHAPE;
  }
  return CP_OK;
}

size_t cp_attn_workspace_bytes(const cp_cache *cache, const cp_attn_args *args) {
  if (check_attn(cache, args) != CP_OK) return 0;
  return attn_workspace_bytes(*cache, *args, plan_attention(*cache, *args, true));
}

int cp_attn_chunk_with_past(const cp_cache *cache, const cp_attn_args *args, cp_stream_t stream) {
  const int st = check_attn(cache, args);
  if (st != CP_OK) return st;
  return to_status(launch_attention(*cache, *args, static_cast<hipStream_t>(stream)));
}

int cp_attn_chunk_with_past_noalloc(const cp_cache *cache, const cp_attn_args *args,
                                    cp_stream_t stream) {
  int st = check_attn(cache, args);
  if (st != CP_OK) return st;
  // the plan the call would take with an unlimited workspace, and what its splits need
  const size_t need = attn_workspace_bytes(*cache, *args, plan_attention(*cache, *args, true));
  if (need > CP_ATTN_SCRATCH_BYTES) return CP_ERR_SCRATCH;
  cp_attn_args a = *args;
  a.workspace = nullptr;
  a.workspace_bytes = 0;
  if (need > 0) {
    st = scratch_on_current_device(&a.workspace);
    if (st != CP_OK) return st;
    a.workspace_bytes = CP_ATTN_SCRATCH_BYTES;
  }
  return to_status(launch_attention(*cache, a, static_cast<hipStream_t>(stream)));
}

int cp_build_mask(float *mask, int64_t ld, const cp_cache *cache, const int32_t *n_valid, int H,
                  int C, int window, cp_stream_t stream) {
  const int st = check_cache(cache);
  if (st != CP_OK) return st;
  if (ld < 0 || H < 1 || C < 0 || window < 0) return CP_ERR_ARG;
  if (static_cast<size_t>(cache->B) * C * ld == 0) return CP_OK;
  if (!mask) return CP_ERR_ARG;
  return to_status(
      launch_build_mask(mask, ld, *cache, n_valid, H, C, window, static_cast<hipStream_t>(stream)));
}

int cp_select_row(const void *x, void *y, const int32_t *idx, int offset, int B, int H, int C,
                  int D, int dtype, cp_stream_t stream) {
  if (dtype != CP_F32 && dtype != CP_BF16) return CP_ERR_DTYPE;
  if (B < 0 || H < 0 || C < 0 || D < 1) return CP_ERR_ARG;
  if (static_cast<size_t>(B) * H == 0) return CP_OK;
  if (!y || !idx || (C > 0 && !x)) return CP_ERR_ARG;
  return to_status(
      launch_select(x, y, idx, offset, B, H, C, D, dtype, static_cast<hipStream_t>(stream)));
}

size_t cp_gdn_workspace_bytes(int B, int H, int P, int dk, int dv) {
  if (B < 0 || H < 0 || P < 0 || !gdn_dims_supported(dk, dv)) return 0;
  return gdn_workspace_bytes(B, H, P, dk, dv);
}

int cp_gdn_chunk_prefill(const float *q, const float *k, const float *v, const float *beta,
                         const float *alpha, float *state, float *out, int B, int H, int P,
                         int dk, int dv, void *workspace, size_t workspace_bytes,
                         cp_stream_t stream) {
  if (B < 0 || H < 0 || P < 0) return CP_ERR_ARG;
  if (!gdn_dims_supported(dk, dv) || !gdn_grid_fits(B, H, P)) return CP_ERR_SHAPE;
  if (static_cast<size_t>(B) * H * P == 0) return CP_OK;  // empty: pointers may be NULL
  if (!q || !k || !v || !beta || !alpha || !state || !out || !workspace) return CP_ERR_ARG;
  const uintptr_t vec = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) |
                        reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(workspace);
  if (vec & 15) return CP_ERR_ARG;  // read and written as 16-byte vectors
  if (workspace_bytes < gdn_workspace_bytes(B, H, P, dk, dv)) return CP_ERR_WORKSPACE;
  return to_status(launch_gdn(q, k, v, beta, alpha, state, out, B, H, P, dk, dv, workspace,
                              static_cast<hipStream_t>(stream)));
}

}  // extern "C"
