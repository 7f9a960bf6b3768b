// Host side of the C ABI: argument validation, workspace sizing, launch
// planning.  Nothing here allocates, frees or synchronises.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/dsa.h"
#include "kernels.h"

namespace {

thread_local char g_err[512] = "";

dsa_status fail(dsa_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int key_token_bytes(int fmt) {
  return fmt == DSA_KEY_FP8 ? 132 : fmt == DSA_KEY_MXFP4 ? 68 : fmt == DSA_KEY_NVFP4 ? 72 : 0;
}
// bytes per latent row inside a page (the row's data padded to whole 128-byte lines)
int lat_row_bytes(int fmt) {
  return fmt == DSA_LAT_BF16 ? 1152 : fmt == DSA_LAT_FP8 ? 640 : fmt == DSA_LAT_NVFP4 ? 384 : 0;
}

dsa_status check_cache(const dsa_cache& c, int token_bytes, const char* what) {
  if (token_bytes == 0) return fail(DSA_ERR_UNSUPPORTED, "%s: unknown format %d", what, c.fmt);
  if (!c.base || !aligned(c.base, 16)) return fail(DSA_ERR_INVALID_ARG, "%s: base null or not 16-byte aligned", what);
  if (c.page_size_log2 < 4 || c.page_size_log2 > 24)
    return fail(DSA_ERR_INVALID_ARG, "%s: page_size_log2 %d outside [4, 24]", what, c.page_size_log2);
  if (c.num_pages < 1) return fail(DSA_ERR_INVALID_ARG, "%s: num_pages < 1", what);
  const int64_t need = (int64_t(1) << c.page_size_log2) * token_bytes;
  if (c.page_bytes % 16 != 0 || c.page_bytes < need)
    return fail(DSA_ERR_INVALID_ARG, "%s: page_bytes %lld not a multiple of 16 or below %lld", what,
                (long long)c.page_bytes, (long long)need);
  return DSA_OK;
}

dsa_status check_batch(const dsa_batch& b, int plog2, bool need_meta) {
  if (b.num_requests < 1 || b.num_rows < 1) return fail(DSA_ERR_INVALID_ARG, "batch: empty batch");
  if (b.max_vis < 1 || b.max_rows_per_req < 1) return fail(DSA_ERR_INVALID_ARG, "batch: max_vis/max_rows_per_req < 1");
  if (!b.tok_vis) return fail(DSA_ERR_INVALID_ARG, "batch: tok_vis is null");
  if (need_meta && !b.req_row_start) return fail(DSA_ERR_INVALID_ARG, "batch: req_row_start is null");
  if (b.block_table) {
    const int64_t pages = ((int64_t)b.max_vis + (int64_t(1) << plog2) - 1) >> plog2;
    if (b.bt_stride < pages)
      return fail(DSA_ERR_INVALID_ARG, "batch: bt_stride %d below the %lld pages max_vis needs", b.bt_stride,
                  (long long)pages);
  } else if ((int64_t)b.max_vis > (int64_t(1) << plog2)) {
    return fail(DSA_ERR_INVALID_ARG, "batch: non-paged cache needs page size >= max_vis");
  }
  return DSA_OK;
}

// ---- top-k plan
struct TopkPlan {
  int cand_cap, slice, nslices, slice_cap;
  size_t off_ctr, off_cand, off_info, total;
};
// Long rows are filtered in slices of 8192 scores; every slice writes its
// candidates to a region of its own of slice_cap entries (8 bytes each), so
// the row's workgroups share no counter.  A slice with more candidates than
// its region sends the row to the finalize's whole-row selection (the
// threshold expects about 2900 of a row's candidates, about 90 per slice at
// 256K scores).
TopkPlan plan_topk(int T, int max_vis, int k) {
  (void)k;
  TopkPlan pl;
  pl.cand_cap = std::min(max_vis, dsa::kTopkFinalCap);
  pl.slice = 8192;
  pl.nslices = (max_vis + pl.slice - 1) / pl.slice;
  pl.slice_cap = std::min(pl.cand_cap, 1024);
  size_t off = 0;
  pl.off_ctr = off;
  off = align_up(off + (size_t)T * 16, 256);
  pl.off_cand = off;
  off = align_up(off + (size_t)T * pl.nslices * pl.slice_cap * 8, 256);
  pl.off_info = off;
  off = align_up(off + (size_t)T * pl.nslices * 8, 256);
  pl.total = off;
  return pl;
}

// ---- sharded top-k plan
struct ShardedPlan {
  int W, T, k, cand, max_local;
  TopkPlan local;
  size_t off_lvis, off_lvis2, off_lidx, off_topk, off_xbuf, off_xcnt, off_flags, off_rowflag, total;
};
ShardedPlan plan_sharded(const dsa_topk_sharded_args& a) {
  ShardedPlan pl;
  pl.W = a.num_shards;
  pl.T = a.num_rows;
  pl.k = a.k;
  pl.cand = a.cand > 0 ? a.cand : std::min(a.k, (3 * a.k + 2 * a.num_shards - 1) / (2 * a.num_shards));
  pl.max_local = std::max(1, (a.max_vis + a.num_shards - 1) / a.num_shards);
  const size_t n = (size_t)pl.W * pl.T;
  pl.local = plan_topk((int)n, pl.max_local, a.k);
  size_t off = 0;
  pl.off_lvis = off;
  off = align_up(off + n * 4, 256);
  pl.off_lvis2 = off;
  off = align_up(off + n * 4, 256);
  pl.off_lidx = off;
  off = align_up(off + n * a.k * 4, 256);
  pl.off_topk = off;
  off = align_up(off + pl.local.total, 256);
  pl.off_xbuf = off;
  off = align_up(off + n * a.k * 8, 256);
  pl.off_xcnt = off;
  off = align_up(off + n * 4, 256);
  pl.off_flags = off;
  off = align_up(off + n * 4, 256);
  pl.off_rowflag = off;
  off = align_up(off + (size_t)pl.T * 4, 256);
  pl.total = off;
  return pl;
}

bool sharded_shape_ok(const dsa_topk_sharded_args& a) {
  return a.num_rows >= 1 && a.num_shards >= 1 && a.num_shards <= dsa::kMaxShards && a.k >= 1 &&
         a.k <= DSA_MAX_TOPK && a.cand >= 0 && a.cand <= a.k && a.max_vis >= 1 &&
         (int64_t)a.num_rows * a.num_shards <= 65535LL * 64;
}

// ---- MLA plan
struct MlaPlan {
  int Hpad, ntiles, nsplit, split_len;
  size_t off_po, off_pl, total;
};
// Keys per workgroup of the multi-row indexer (a request's rows are staged
// once per workgroup): the multiple of the 256-key round, at most 4096 keys
// (the staged page ids), that finishes first when the requests' chunks run in
// waves of per_cu workgroups per CU on 256 CUs -- waves x (chunk + 256), the
// 256 standing for a workgroup's start-up -- so a chunk that leaves a few
// workgroups for a second, partial wave is not taken.
int multi_row_chunk(int max_vis, int num_requests, int per_cu) {
  const int64_t slots = (int64_t)per_cu * 256;
  int best = 4096;
  int64_t best_cost = INT64_MAX;
  for (int chunk = 256; chunk <= 4096; chunk += 256) {
    const int64_t n = (int64_t)num_requests * ((max_vis + chunk - 1) / chunk);
    const int64_t cost = (n + slots - 1) / slots * (chunk + 256);
    if (cost < best_cost) {
      best_cost = cost;
      best = chunk;
    }
  }
  return best;
}

MlaPlan plan_mla(const dsa_mla_args& a, bool prefill, int max_splits = 64) {
  MlaPlan pl;
  pl.Hpad = (a.num_heads + 15) / 16 * 16;
  pl.ntiles = pl.Hpad / 16;
  int want;
  if (prefill) {
    want = 1;
  } else if (a.num_splits > 0) {
    want = a.num_splits;
  } else {
    // Fill the resident workgroup slots in one round; a second, partial round
    // would cost a whole extra pass.
    const dsa::MlaShape sh = dsa::mla_shape(pl.ntiles, a.latents.fmt == DSA_LAT_NVFP4);
    const int64_t resident = 256 * sh.resident_per_cu;
    const int64_t per_split = (int64_t)a.num_rows * sh.groups;
    want = (int)std::min<int64_t>(64, std::max<int64_t>(1, resident / per_split));
    want = std::min(want, max_splits);
  }
  want = std::max(1, std::min({want, (a.k + 15) / 16, 64}));
  pl.split_len = ((a.k + want - 1) / want + 15) / 16 * 16;
  pl.nsplit = (a.k + pl.split_len - 1) / pl.split_len;
  size_t off = 0;
  pl.off_po = 0;
  pl.off_pl = 0;
  if (pl.nsplit > 1) {
    off = align_up((size_t)a.num_rows * pl.nsplit * a.num_heads * 512 * 4, 256);
    pl.off_pl = off;
    off = align_up(off + (size_t)a.num_rows * pl.nsplit * a.num_heads * 4, 256);
  }
  pl.total = off;
  return pl;
}

dsa_status check_mla(const dsa_mla_args* a) {
  if (!a) return fail(DSA_ERR_INVALID_ARG, "mla: null args");
  if (a->num_rows < 1) return fail(DSA_ERR_INVALID_ARG, "mla: num_rows < 1");
  if (a->num_heads < 1 || a->num_heads > DSA_MAX_HEADS) return fail(DSA_ERR_INVALID_ARG, "mla: num_heads %d", a->num_heads);
  if (a->k < 1 || a->k > DSA_MAX_TOPK) return fail(DSA_ERR_INVALID_ARG, "mla: k %d outside [1, 2048]", a->k);
  if (!a->q || !aligned(a->q, 16)) return fail(DSA_ERR_INVALID_ARG, "mla: q null or not 16-byte aligned");
  if (!a->rows) return fail(DSA_ERR_INVALID_ARG, "mla: rows is null");
  if (!a->out || !aligned(a->out, 16)) return fail(DSA_ERR_INVALID_ARG, "mla: out null or not 16-byte aligned");
  if (!(std::isfinite(a->sm_scale) && a->sm_scale > 0.f)) return fail(DSA_ERR_INVALID_ARG, "mla: sm_scale");
  if (a->num_splits < 0 || a->num_splits > DSA_MAX_TOPK / 16) return fail(DSA_ERR_INVALID_ARG, "mla: num_splits");
  return check_cache(a->latents, lat_row_bytes(a->latents.fmt), "mla latents");
}

// Split count of an allocation-free decode call: the automatic count,
// lowered until the partials fit the device scratch (an explicit count is
// kept and checked by the caller).
MlaPlan plan_mla_in_scratch(const dsa_mla_args& a) {
  MlaPlan pl = plan_mla(a, false);
  for (int cap = pl.nsplit - 1; a.num_splits == 0 && pl.total > dsa::kMlaScratchBytes && cap >= 1; --cap)
    pl = plan_mla(a, false, cap);
  return pl;
}

// scratch != NULL: the partials go to that device scratch (the
// allocation-free entry point), and the workspace arguments are ignored.
dsa_status run_mla(const dsa_mla_args* a, hipStream_t stream, bool prefill, void* scratch = nullptr) {
  dsa_status st = check_mla(a);
  if (st != DSA_OK) return st;
  const MlaPlan pl = scratch ? plan_mla_in_scratch(*a) : plan_mla(*a, prefill);
  if (scratch) {
    if (pl.total > dsa::kMlaScratchBytes)
      return fail(DSA_ERR_WORKSPACE, "mla_noalloc: %d splits need %zu bytes of partials, above the %zu-byte scratch",
                  pl.nsplit, pl.total, dsa::kMlaScratchBytes);
  } else if (pl.total > 0) {
    if (!a->workspace || !aligned(a->workspace, 256))
      return fail(DSA_ERR_WORKSPACE, "mla: workspace null or not 256-byte aligned (%zu bytes needed)", pl.total);
    if (a->workspace_bytes < pl.total)
      return fail(DSA_ERR_WORKSPACE, "mla: workspace %zu bytes, %zu needed", a->workspace_bytes, pl.total);
  }
  dsa::MlaParams p{};
  p.T = a->num_rows;
  p.H = a->num_heads;
  p.Hpad = pl.Hpad;
  p.ntiles = pl.ntiles;
  p.q = static_cast<const __bf16*>(a->q);
  p.lat = static_cast<const uint8_t*>(a->latents.base);
  p.page_bytes = a->latents.page_bytes;
  p.plog2 = a->latents.page_size_log2;
  p.num_pages = a->latents.num_pages;
  p.fmt = a->latents.fmt;
  p.rows = a->rows;
  p.k = a->k;
  p.sm_log2 = a->sm_scale * 1.4426950408889634f;
  p.nsplit = pl.nsplit;
  p.split_len = pl.split_len;
  p.prefill = prefill ? 1 : 0;
  p.out = a->out;
  p.lse = a->lse;
  char* ws = static_cast<char*>(scratch ? scratch : a->workspace);
  p.part_o = pl.nsplit > 1 ? reinterpret_cast<float*>(ws + pl.off_po) : nullptr;
  p.part_lse = pl.nsplit > 1 ? reinterpret_cast<float*>(ws + pl.off_pl) : nullptr;
  st = dsa::launch_mla(p, stream);
  if (st != DSA_OK) return fail(st, "mla: launch failed: %s", hipGetErrorString(hipGetLastError()));
  return DSA_OK;
}

}  // namespace

extern "C" {

int32_t dsa_abi_version(void) { return DSA_ABI_VERSION; }

int32_t dsa_check_debug_flag(void) {
#if DSA_DEBUG
  if (hipDeviceSynchronize() != hipSuccess) return -1;
  const uint32_t v = dsa::debug_take_indexer() | dsa::debug_take_indexer_fp8() | dsa::debug_take_topk() |
                     dsa::debug_take_mla() | dsa::debug_take_quant() | dsa::debug_take_merge() |
                     dsa::debug_take_msa();
  return (int32_t)v;
#else
  return -1;
#endif
}

const char* dsa_last_error(void) { return g_err; }

const char* dsa_status_str(dsa_status s) {
  switch (s) {
    case DSA_OK: return "DSA_OK";
    case DSA_ERR_INVALID_ARG: return "DSA_ERR_INVALID_ARG";
    case DSA_ERR_UNSUPPORTED: return "DSA_ERR_UNSUPPORTED";
    case DSA_ERR_WORKSPACE: return "DSA_ERR_WORKSPACE";
    case DSA_ERR_HIP: return "DSA_ERR_HIP";
  }
  return "DSA_ERR_UNKNOWN";
}

dsa_status dsa_indexer_scores(const dsa_indexer_args* a, hipStream_t stream) {
  g_err[0] = 0;
  if (!a) return fail(DSA_ERR_INVALID_ARG, "indexer: null args");
  dsa_status st = check_cache(a->keys, key_token_bytes(a->keys.fmt), "indexer keys");
  if (st != DSA_OK) return st;
  st = check_batch(a->batch, a->keys.page_size_log2, true);
  if (st != DSA_OK) return st;
  if (!a->q || !aligned(a->q, 16)) return fail(DSA_ERR_INVALID_ARG, "indexer: q null or not 16-byte aligned");
  if (!a->w || !aligned(a->w, 16)) return fail(DSA_ERR_INVALID_ARG, "indexer: w null or not 16-byte aligned");
  if (!a->scores || !aligned(a->scores, 16)) return fail(DSA_ERR_INVALID_ARG, "indexer: scores null or not 16-byte aligned");
  if (a->ld < a->batch.max_vis || a->ld % 4 != 0) return fail(DSA_ERR_INVALID_ARG, "indexer: ld %lld", (long long)a->ld);
  if (a->batch.num_requests > 65535) return fail(DSA_ERR_INVALID_ARG, "indexer: more than 65535 requests");
  if (a->q_fmt == DSA_Q_FP8 && (int64_t)a->batch.max_rows_per_req > 16 * 65535)
    return fail(DSA_ERR_INVALID_ARG, "indexer: too many rows per request");
  if (a->q_fmt != DSA_Q_BF16 && a->q_fmt != DSA_Q_FP8 && a->q_fmt != DSA_Q_MXFP4)
    return fail(DSA_ERR_UNSUPPORTED, "indexer: q_fmt %d", a->q_fmt);
  if (a->q_fmt == DSA_Q_FP8 && a->keys.fmt != DSA_KEY_FP8)
    return fail(DSA_ERR_UNSUPPORTED, "indexer: FP8 q runs against FP8 keys only");
  if (a->q_fmt == DSA_Q_MXFP4 && a->keys.fmt != DSA_KEY_MXFP4)
    return fail(DSA_ERR_UNSUPPORTED, "indexer: MXFP4 q runs against MXFP4 keys only");
  if (a->q_fmt == DSA_Q_FP8 && (!a->q_scale || !aligned(a->q_scale, 16)))
    return fail(DSA_ERR_INVALID_ARG, "indexer: FP8 q needs a 16-byte aligned q_scale");
  if (a->q_fmt == DSA_Q_MXFP4 && !a->q_scale)
    return fail(DSA_ERR_INVALID_ARG, "indexer: MXFP4 q needs its E8M0 scales (q_scale)");

  dsa::IndexerParams p{};
  const dsa_batch& b = a->batch;
  p.R = b.num_requests;
  p.T = b.num_rows;
  p.req_row_start = b.req_row_start;
  p.tok_req = b.tok_req;
  p.tok_vis = b.tok_vis;
  p.block_table = b.block_table;
  p.bt_stride = b.bt_stride;
  p.max_vis = b.max_vis;
  p.keys = static_cast<const uint8_t*>(a->keys.base);
  p.page_bytes = a->keys.page_bytes;
  p.plog2 = a->keys.page_size_log2;
  p.num_pages = a->keys.num_pages;
  p.key_fmt = a->keys.fmt;
  p.w = a->w;
  p.scores = a->scores;
  p.ld = a->ld;
  if (a->q_fmt == DSA_Q_MXFP4) {
    p.q8 = static_cast<const uint8_t*>(a->q);
    p.q_e8m0 = static_cast<const uint8_t*>(a->q_scale);
    // keys per workgroup as for single-row BF16 requests (the streaming kernel)
    const int64_t target = (int64_t)b.max_vis * b.num_requests / 2048;
    int chunk = 256;
    while (chunk < dsa::kIndexerRowChunkFp4 && chunk * 2 <= target) chunk *= 2;
    p.chunk = chunk;
    p.max_rows_per_req = b.max_rows_per_req;
    st = dsa::launch_indexer_bf16(p, stream);
  } else if (a->q_fmt == DSA_Q_BF16) {
    p.q = static_cast<const __bf16*>(a->q);
    if (b.max_rows_per_req == 1) {
      // keys per workgroup: single-row requests stream keys and want many
      // workgroups in flight (about 2048)
      const int64_t target = (int64_t)b.max_vis * b.num_requests / 2048;
      const int cap = a->keys.fmt == DSA_KEY_FP8 ? dsa::kIndexerRowChunkFp8 : dsa::kIndexerRowChunkFp4;
      int chunk = 256;
      while (chunk < cap && chunk * 2 <= target) chunk *= 2;
      p.chunk = chunk;
    } else {
      // multi-row requests stage their rows once per workgroup, so fewer,
      // longer workgroups (about 512, two per CU) amortise that
      const int64_t target = (int64_t)b.max_vis * b.num_requests / 512;
      int chunk = 256;
      while (chunk < 4096 && chunk * 2 <= target) chunk *= 2;
      p.chunk = chunk;
    }
    p.qrows = std::min(b.max_rows_per_req, dsa::kIndexerMaxRowsPerPass);
    p.max_rows_per_req = b.max_rows_per_req;
    st = dsa::launch_indexer_bf16(p, stream);
  } else if (b.max_rows_per_req <= dsa::kIndexerQ8MaxRows) {
    // FP8 q of few-row (decode) requests: the multi-row kernel on the FP8
    // instruction, keys read raw; workgroups as for BF16 multi-row requests
    p.q8 = static_cast<const uint8_t*>(a->q);
    p.q_scale = static_cast<const float*>(a->q_scale);
    p.chunk = multi_row_chunk(b.max_vis, b.num_requests, 3);  // three waves per SIMD
    p.qrows = std::min(b.max_rows_per_req, dsa::kIndexerMaxRowsPerPass);
    p.max_rows_per_req = b.max_rows_per_req;
    st = dsa::launch_indexer_bf16(p, stream);
  } else {
    p.q8 = static_cast<const uint8_t*>(a->q);
    p.q_scale = static_cast<const float*>(a->q_scale);
    p.max_rows_per_req = b.max_rows_per_req;
    // key segment per workgroup: about 2048 workgroups over rows x keys
    const int64_t row_groups = (int64_t)b.num_requests * ((b.max_rows_per_req + 15) / 16);
    int chunk = 256;
    while (chunk < 16384 && row_groups * (((int64_t)b.max_vis + 2 * chunk - 1) / (2 * chunk)) >= 2048) chunk *= 2;
    p.chunk = chunk;
    st = dsa::launch_indexer_fp8(p, stream);
  }
  if (st != DSA_OK) return fail(st, "indexer: launch failed: %s", hipGetErrorString(hipGetLastError()));
  return DSA_OK;
}

namespace {
struct PrefixPlan {
  int npfx, ns_max;
  size_t off_vis1, off_vis2, off_sub, off_src, off_ptab, total;
};
PrefixPlan plan_prefix(const dsa_indexer_prefix_args& a) {
  PrefixPlan pl;
  const int P = 1 << a.base.keys.page_size_log2;
  const int T = a.base.batch.num_rows;
  pl.npfx = a.prefix_len / P;
  // every group adds at most one partial sub-group
  pl.ns_max = std::max(1, a.num_groups) + (T + dsa::kPrefixSubRows - 1) / dsa::kPrefixSubRows;
  size_t off = 0;
  pl.off_vis1 = off;
  off = align_up(off + (size_t)T * 4, 256);
  pl.off_vis2 = off;
  off = align_up(off + (size_t)T * 4, 256);
  pl.off_sub = off;
  off = align_up(off + (size_t)(pl.ns_max + 1) * 4, 256);
  pl.off_src = off;
  off = align_up(off + (size_t)pl.ns_max * 4, 256);
  pl.off_ptab = off;
  off = align_up(off + (size_t)pl.ns_max * std::max(1, pl.npfx) * 4, 256);
  pl.total = off;
  return pl;
}
}  // namespace

dsa_status dsa_indexer_scores_prefix(const dsa_indexer_prefix_args* a, hipStream_t stream) {
  g_err[0] = 0;
  if (!a) return fail(DSA_ERR_INVALID_ARG, "indexer_prefix: null args");
  const dsa_indexer_args& base = a->base;
  dsa_status st = check_cache(base.keys, key_token_bytes(base.keys.fmt), "indexer keys");
  if (st != DSA_OK) return st;
  st = check_batch(base.batch, base.keys.page_size_log2, true);
  if (st != DSA_OK) return st;
  if (base.q_fmt != DSA_Q_BF16) return fail(DSA_ERR_UNSUPPORTED, "indexer_prefix: BF16 q only");
  if (!base.batch.block_table) return fail(DSA_ERR_INVALID_ARG, "indexer_prefix: a block table is required");
  const int P = 1 << base.keys.page_size_log2;
  if (a->num_groups < 1 || a->num_groups > base.batch.num_requests || !a->group_row_start || !a->group_first_req ||
      a->max_rows_per_group < 1)
    return fail(DSA_ERR_INVALID_ARG, "indexer_prefix: bad group description");
  if (a->prefix_len < 0 || a->prefix_len % P != 0 || a->prefix_len > base.batch.max_vis)
    return fail(DSA_ERR_INVALID_ARG, "indexer_prefix: prefix_len %d (multiple of %d, at most max_vis)", a->prefix_len, P);
  if (!base.scores || !aligned(base.scores, 16) || base.ld % 4 != 0 || base.ld < base.batch.max_vis)
    return fail(DSA_ERR_INVALID_ARG, "indexer_prefix: scores / ld");
  const PrefixPlan pl = plan_prefix(*a);
  if (!a->workspace || !aligned(a->workspace, 256))
    return fail(DSA_ERR_WORKSPACE, "indexer_prefix: workspace null or not 256-byte aligned (%zu bytes needed)", pl.total);
  if (a->workspace_bytes < pl.total)
    return fail(DSA_ERR_WORKSPACE, "indexer_prefix: workspace %zu bytes, %zu needed", a->workspace_bytes, pl.total);
  char* ws = static_cast<char*>(a->workspace);
  int32_t* vis1 = reinterpret_cast<int32_t*>(ws + pl.off_vis1);
  int32_t* vis2 = reinterpret_cast<int32_t*>(ws + pl.off_vis2);
  int32_t* ptab = reinterpret_cast<int32_t*>(ws + pl.off_ptab);
  int32_t* sub_start = reinterpret_cast<int32_t*>(ws + pl.off_sub);
  int32_t* sub_src = reinterpret_cast<int32_t*>(ws + pl.off_src);
  const int L = a->prefix_len;
  st = dsa::launch_prefix_prep(base.batch.tok_vis, base.batch.num_rows, base.batch.max_vis, L, base.batch.block_table,
                               base.batch.bt_stride, base.batch.num_requests, a->group_row_start, a->group_first_req,
                               a->num_groups, pl.ns_max, pl.npfx, sub_start, sub_src, vis1, vis2, ptab, stream);
  if (st != DSA_OK) return fail(st, "indexer_prefix: launch failed: %s", hipGetErrorString(hipGetLastError()));
  if (L > 0) {  // shared pages, once per group for all of its rows
    dsa_indexer_args a1 = base;
    a1.batch.num_requests = pl.ns_max;  // sub-groups of at most kPrefixSubRows rows (empty ones at the end)
    a1.batch.req_row_start = sub_start;
    a1.batch.tok_vis = vis1;
    a1.batch.block_table = ptab;
    a1.batch.bt_stride = pl.npfx;
    a1.batch.max_vis = L;
    a1.batch.max_rows_per_req = std::min(a->max_rows_per_group, dsa::kPrefixSubRows);
    st = dsa_indexer_scores(&a1, stream);
    if (st != DSA_OK) return st;
  }
  if (base.batch.max_vis > L) {  // every request's own pages past the prefix
    dsa_indexer_args a2 = base;
    a2.batch.tok_vis = vis2;
    a2.batch.block_table = base.batch.block_table + L / P;
    a2.batch.bt_stride = base.batch.bt_stride;
    a2.batch.max_vis = base.batch.max_vis - L;
    a2.scores = base.scores + L;
    st = dsa_indexer_scores(&a2, stream);
    if (st != DSA_OK) return st;
  }
  return DSA_OK;
}

dsa_status dsa_topk(const dsa_topk_args* a, hipStream_t stream) {
  g_err[0] = 0;
  if (!a) return fail(DSA_ERR_INVALID_ARG, "topk: null args");
  const dsa_batch& b = a->batch;
  if (a->k < 1 || a->k > DSA_MAX_TOPK) return fail(DSA_ERR_INVALID_ARG, "topk: k %d outside [1, 2048]", a->k);
  if (b.num_rows < 1 || b.max_vis < 1 || !b.tok_vis) return fail(DSA_ERR_INVALID_ARG, "topk: bad batch");
  if (!a->scores || !aligned(a->scores, 16)) return fail(DSA_ERR_INVALID_ARG, "topk: scores null or not 16-byte aligned");
  if (a->ld < b.max_vis || a->ld % 4 != 0) return fail(DSA_ERR_INVALID_ARG, "topk: ld %lld", (long long)a->ld);
  if (!a->idx) return fail(DSA_ERR_INVALID_ARG, "topk: idx is null");
  if (a->rows) {
    if (a->page_size_log2 < 4 || a->page_size_log2 > 24) return fail(DSA_ERR_INVALID_ARG, "topk: page_size_log2");
    if (a->num_pages < 1 || ((int64_t)a->num_pages << a->page_size_log2) > INT32_MAX)
      return fail(DSA_ERR_INVALID_ARG, "topk: num_pages %d (rows of the pool must fit int32)", a->num_pages);
    if (!b.tok_req) return fail(DSA_ERR_INVALID_ARG, "topk: rows need tok_req");
    dsa_status st = check_batch(b, a->page_size_log2, false);
    if (st != DSA_OK) return st;
  }
  if (b.num_rows > 65535 * 64) return fail(DSA_ERR_INVALID_ARG, "topk: too many rows");
  const TopkPlan pl = plan_topk(b.num_rows, b.max_vis, a->k);
  if (!a->workspace || !aligned(a->workspace, 256))
    return fail(DSA_ERR_WORKSPACE, "topk: workspace null or not 256-byte aligned (%zu bytes needed)", pl.total);
  if (a->workspace_bytes < pl.total)
    return fail(DSA_ERR_WORKSPACE, "topk: workspace %zu bytes, %zu needed", a->workspace_bytes, pl.total);
  dsa::TopkParams p{};
  p.T = b.num_rows;
  p.scores = a->scores;
  p.ld = a->ld;
  p.tok_vis = b.tok_vis;
  p.tok_req = b.tok_req;
  p.R = b.num_requests;
  p.max_vis = b.max_vis;
  p.k = a->k;
  p.block_table = b.block_table;
  p.bt_stride = b.bt_stride;
  p.plog2 = a->page_size_log2;
  p.num_pages = a->num_pages;
  p.idx = a->idx;
  p.rows = a->rows;
  p.count = a->count;
  char* ws = static_cast<char*>(a->workspace);
  p.ctr = reinterpret_cast<uint32_t*>(ws + pl.off_ctr);
  p.cand = reinterpret_cast<uint32_t*>(ws + pl.off_cand);
  p.slice_info = reinterpret_cast<uint32_t*>(ws + pl.off_info);
  p.cand_cap = pl.cand_cap;
  p.slice_cap = pl.slice_cap;
  p.slice = pl.slice;
  p.nslices = pl.nslices;
  dsa_status st = dsa::launch_topk(p, stream);
  if (st != DSA_OK) return fail(st, "topk: launch failed: %s", hipGetErrorString(hipGetLastError()));
  return DSA_OK;
}

dsa_status dsa_topk_sharded(const dsa_topk_sharded_args* a, hipStream_t stream) {
  g_err[0] = 0;
  if (!a) return fail(DSA_ERR_INVALID_ARG, "topk_sharded: null args");
  if (!sharded_shape_ok(*a))
    return fail(DSA_ERR_INVALID_ARG, "topk_sharded: rows %d, shards %d (1..%d), k %d, cand %d or max_vis %d out of range",
                a->num_rows, a->num_shards, dsa::kMaxShards, a->k, a->cand, a->max_vis);
  if (!a->scores || !aligned(a->scores, 16))
    return fail(DSA_ERR_INVALID_ARG, "topk_sharded: scores null or not 16-byte aligned");
  const int64_t max_local = (a->max_vis + a->num_shards - 1) / a->num_shards;
  if (a->ld < max_local || a->ld % 4 != 0)
    return fail(DSA_ERR_INVALID_ARG, "topk_sharded: ld %lld (needs >= %lld, multiple of 4)", (long long)a->ld,
                (long long)max_local);
  if (!a->tok_vis || !a->idx) return fail(DSA_ERR_INVALID_ARG, "topk_sharded: tok_vis or idx is null");
  const ShardedPlan pl = plan_sharded(*a);
  if (!a->workspace || !aligned(a->workspace, 256))
    return fail(DSA_ERR_WORKSPACE, "topk_sharded: workspace null or not 256-byte aligned (%zu bytes needed)", pl.total);
  if (a->workspace_bytes < pl.total)
    return fail(DSA_ERR_WORKSPACE, "topk_sharded: workspace %zu bytes, %zu needed", a->workspace_bytes, pl.total);
  char* ws = static_cast<char*>(a->workspace);
  dsa::MergeParams m{};
  m.T = pl.T;
  m.W = pl.W;
  m.k = pl.k;
  m.cand = pl.cand;
  m.scores = a->scores;
  m.ld = a->ld;
  m.tok_vis = a->tok_vis;
  m.max_vis = a->max_vis;
  m.idx = a->idx;
  m.count = a->count;
  m.lvis = reinterpret_cast<int32_t*>(ws + pl.off_lvis);
  m.lvis2 = reinterpret_cast<int32_t*>(ws + pl.off_lvis2);
  m.lidx = reinterpret_cast<int32_t*>(ws + pl.off_lidx);
  m.xbuf = reinterpret_cast<uint64_t*>(ws + pl.off_xbuf);
  m.xcnt = reinterpret_cast<int32_t*>(ws + pl.off_xcnt);
  m.flags = a->resend ? a->resend : reinterpret_cast<int32_t*>(ws + pl.off_flags);
  m.rowflag = reinterpret_cast<int32_t*>(ws + pl.off_rowflag);
  dsa::TopkParams p{};
  p.T = pl.W * pl.T;
  p.scores = a->scores;
  p.ld = a->ld;
  p.tok_vis = m.lvis;
  p.max_vis = pl.max_local;
  p.k = a->k;
  p.idx = m.lidx;
  char* tws = ws + pl.off_topk;
  p.ctr = reinterpret_cast<uint32_t*>(tws + pl.local.off_ctr);
  p.cand = reinterpret_cast<uint32_t*>(tws + pl.local.off_cand);
  p.slice_info = reinterpret_cast<uint32_t*>(tws + pl.local.off_info);
  p.cand_cap = pl.local.cand_cap;
  p.slice_cap = pl.local.slice_cap;
  p.slice = pl.local.slice;
  p.nslices = pl.local.nslices;
  p.skip_empty = 1;
  dsa_status st = dsa::launch_topk_sharded(m, p, stream);
  if (st != DSA_OK) return fail(st, "topk_sharded: launch failed: %s", hipGetErrorString(hipGetLastError()));
  return DSA_OK;
}

dsa_status dsa_msa_decode(const dsa_msa_args* a, hipStream_t stream) {
  g_err[0] = 0;
  if (!a) return fail(DSA_ERR_INVALID_ARG, "msa: null args");
  const dsa_batch& b = a->batch;
  if (a->num_kv_heads < 1 || a->num_kv_heads > 8) return fail(DSA_ERR_INVALID_ARG, "msa: Hkv %d outside [1, 8]", a->num_kv_heads);
  if (a->num_q_heads < a->num_kv_heads || a->num_q_heads % a->num_kv_heads != 0 ||
      a->num_q_heads / a->num_kv_heads > 16)
    return fail(DSA_ERR_INVALID_ARG, "msa: Hq %d must be a multiple of Hkv %d with at most 16 per group",
                a->num_q_heads, a->num_kv_heads);
  if (a->top_blocks < 1 || a->top_blocks > 16) return fail(DSA_ERR_INVALID_ARG, "msa: top_blocks %d", a->top_blocks);
  if (!b.block_table) return fail(DSA_ERR_INVALID_ARG, "msa: a block table is required");
  dsa_status st = check_batch(b, 7, true);
  if (st != DSA_OK) return st;
  if (!b.tok_req) return fail(DSA_ERR_INVALID_ARG, "msa: tok_req is null");
  if (a->num_blocks < 1) return fail(DSA_ERR_INVALID_ARG, "msa: num_blocks < 1");
  if (!a->index_keys || !aligned(a->index_keys, 16) || !a->kv || !aligned(a->kv, 16) || !a->q_idx ||
      !aligned(a->q_idx, 16) || !a->q || !aligned(a->q, 16) || !a->sel_blocks || !a->out)
    return fail(DSA_ERR_INVALID_ARG, "msa: null or unaligned pointer");
  if (b.num_rows > 65535 * 64 / 8) return fail(DSA_ERR_INVALID_ARG, "msa: too many rows");
  const int nblk = (b.max_vis + 127) / 128;
  const size_t off_part = align_up((size_t)b.num_rows * a->num_kv_heads * nblk * 4, 256);
  const size_t need = off_part + align_up((size_t)b.num_rows * a->num_kv_heads * dsa::kMsaSplits *
                                          dsa::kMsaPartFloats * 4, 256);
  if (!a->workspace || !aligned(a->workspace, 256))
    return fail(DSA_ERR_WORKSPACE, "msa: workspace null or not 256-byte aligned (%zu bytes needed)", need);
  if (a->workspace_bytes < need) return fail(DSA_ERR_WORKSPACE, "msa: workspace %zu bytes, %zu needed", a->workspace_bytes, need);
  dsa::MsaParams p{};
  p.R = b.num_requests;
  p.T = b.num_rows;
  p.hkv = a->num_kv_heads;
  p.hq = a->num_q_heads;
  p.G = a->num_q_heads / a->num_kv_heads;
  p.top = a->top_blocks;
  p.nblk_ld = nblk;
  p.req_row_start = b.req_row_start;
  p.tok_req = b.tok_req;
  p.tok_vis = b.tok_vis;
  p.max_vis = b.max_vis;
  p.bt = b.block_table;
  p.bt_stride = b.bt_stride;
  p.pool_blocks = a->num_blocks;
  p.idx_pool = static_cast<const uint8_t*>(a->index_keys);
  p.kv_pool = static_cast<const uint8_t*>(a->kv);
  p.q_idx = static_cast<const __bf16*>(a->q_idx);
  p.q = static_cast<const __bf16*>(a->q);
  p.k_scale = a->k_scale;
  p.v_scale = a->v_scale;
  p.sm_scale = a->sm_scale;
  p.bscore = static_cast<float*>(a->workspace);
  p.part = reinterpret_cast<float*>(static_cast<char*>(a->workspace) + off_part);
  p.sel = a->sel_blocks;
  p.out = a->out;
  p.lse = a->lse;
  st = dsa::launch_msa(p, nblk, stream);
  if (st != DSA_OK) return fail(st, "msa: launch failed: %s", hipGetErrorString(hipGetLastError()));
  return DSA_OK;
}

dsa_status dsa_translate_pages(const int32_t* idx, int32_t k, const dsa_batch* b, int32_t page_size_log2,
                               int32_t num_pages, int32_t* rows, hipStream_t stream) {
  g_err[0] = 0;
  if (!idx || !rows || !b) return fail(DSA_ERR_INVALID_ARG, "translate: null pointer");
  if (k < 1 || k > DSA_MAX_TOPK) return fail(DSA_ERR_INVALID_ARG, "translate: k %d", k);
  if (b->num_rows < 1 || b->num_requests < 1 || !b->tok_req) return fail(DSA_ERR_INVALID_ARG, "translate: bad batch");
  if (page_size_log2 < 4 || page_size_log2 > 24) return fail(DSA_ERR_INVALID_ARG, "translate: page_size_log2");
  if (b->block_table && b->bt_stride < 1) return fail(DSA_ERR_INVALID_ARG, "translate: bt_stride");
  if (num_pages < 1 || ((int64_t)num_pages << page_size_log2) > INT32_MAX)
    return fail(DSA_ERR_INVALID_ARG, "translate: num_pages %d (rows of the pool must fit int32)", num_pages);
  dsa_status st = dsa::launch_translate(idx, k, b->num_rows, b->tok_req, b->num_requests, b->block_table, b->bt_stride,
                                        page_size_log2, num_pages, rows, stream);
  if (st != DSA_OK) return fail(st, "translate: launch failed: %s", hipGetErrorString(hipGetLastError()));
  return DSA_OK;
}

dsa_status sparse_mla_decode(const dsa_mla_args* a, hipStream_t stream) {
  g_err[0] = 0;
  return run_mla(a, stream, false);
}

dsa_status sparse_mla_prefill(const dsa_mla_args* a, hipStream_t stream) {
  g_err[0] = 0;
  return run_mla(a, stream, true);
}

dsa_status sparse_mla_decode_noalloc(const dsa_mla_args* a, hipStream_t stream) {
  g_err[0] = 0;
  dsa_status st = check_mla(a);
  if (st != DSA_OK) return st;
  const MlaPlan pl = plan_mla_in_scratch(*a);
  if (pl.total > dsa::kMlaScratchBytes)
    return fail(DSA_ERR_WORKSPACE, "mla_noalloc: %d splits need %zu bytes of partials, above the %zu-byte scratch",
                pl.nsplit, pl.total, dsa::kMlaScratchBytes);
  void* scratch = nullptr;
  if (dsa::mla_scratch(&scratch) != DSA_OK)
    return fail(DSA_ERR_HIP, "mla_noalloc: the device scratch address could not be resolved: %s",
                hipGetErrorString(hipGetLastError()));
  return run_mla(a, stream, false, scratch);
}

dsa_status dsa_quantize_q(const dsa_quant_q_args* a, hipStream_t stream) {
  g_err[0] = 0;
  if (!a) return fail(DSA_ERR_INVALID_ARG, "quantize_q: null args");
  if (a->num_rows < 0) return fail(DSA_ERR_INVALID_ARG, "quantize_q: num_rows < 0");
  if (a->fmt != DSA_Q_FP8 && a->fmt != DSA_Q_MXFP4) return fail(DSA_ERR_UNSUPPORTED, "quantize_q: fmt %d", a->fmt);
  if (a->num_rows == 0) return DSA_OK;
  if (a->num_rows > 0x7FFFFFFF / 32) return fail(DSA_ERR_INVALID_ARG, "quantize_q: too many rows");
  if (!a->q || !aligned(a->q, 16)) return fail(DSA_ERR_INVALID_ARG, "quantize_q: q null or not 16-byte aligned");
  if (!a->q_out || !aligned(a->q_out, 16)) return fail(DSA_ERR_INVALID_ARG, "quantize_q: q_out null or not 16-byte aligned");
  if (!a->q_scale || (a->fmt == DSA_Q_FP8 && !aligned(a->q_scale, 4)))
    return fail(DSA_ERR_INVALID_ARG, "quantize_q: q_scale null or misaligned");
  if (a->w_folded) {
    if (a->fmt != DSA_Q_FP8) return fail(DSA_ERR_INVALID_ARG, "quantize_q: w_folded is for FP8 rows only");
    if (!a->w || !aligned(a->w, 4) || !aligned(a->w_folded, 4))
      return fail(DSA_ERR_INVALID_ARG, "quantize_q: w_folded needs w (both 4-byte aligned)");
  }
  dsa::QuantQParams p{};
  p.T = a->num_rows;
  p.q = static_cast<const uint16_t*>(a->q);
  p.w = a->w;
  p.fmt = a->fmt;
  p.out = static_cast<uint8_t*>(a->q_out);
  p.scale = a->q_scale;
  p.w_folded = a->w_folded;
  const dsa_status st = dsa::launch_quantize_q(p, stream);
  if (st != DSA_OK) return fail(st, "quantize_q: launch failed: %s", hipGetErrorString(hipGetLastError()));
  return DSA_OK;
}

dsa_status dsa_cache_insert(const dsa_insert_args* a, hipStream_t stream) {
  g_err[0] = 0;
  if (!a) return fail(DSA_ERR_INVALID_ARG, "cache_insert: null args");
  if (a->num_tokens < 0) return fail(DSA_ERR_INVALID_ARG, "cache_insert: num_tokens < 0");
  if (!a->key_vals && !a->lat_vals) return fail(DSA_ERR_INVALID_ARG, "cache_insert: neither keys nor latents given");
  if (a->key_vals) {
    if (a->keys.fmt != DSA_KEY_FP8 && a->keys.fmt != DSA_KEY_MXFP4 && a->keys.fmt != DSA_KEY_NVFP4)
      return fail(DSA_ERR_UNSUPPORTED, "cache_insert: key fmt %d", a->keys.fmt);
    dsa_status st = check_cache(a->keys, key_token_bytes(a->keys.fmt), "cache_insert keys");
    if (st != DSA_OK) return st;
    if (!aligned(a->key_vals, 4)) return fail(DSA_ERR_INVALID_ARG, "cache_insert: key_vals not 4-byte aligned");
  }
  if (a->lat_vals) {
    dsa_status st = check_cache(a->latents, lat_row_bytes(a->latents.fmt), "cache_insert latents");
    if (st != DSA_OK) return st;
    if (!aligned(a->lat_vals, 16)) return fail(DSA_ERR_INVALID_ARG, "cache_insert: lat_vals not 16-byte aligned");
  }
  if (a->key_vals && a->lat_vals && a->keys.page_size_log2 != a->latents.page_size_log2)
    return fail(DSA_ERR_INVALID_ARG, "cache_insert: key and latent pages hold different token counts");
  if (a->num_tokens == 0) return DSA_OK;
  if (a->num_requests < 1) return fail(DSA_ERR_INVALID_ARG, "cache_insert: num_requests < 1");
  if (!a->tok_req || !a->tok_pos) return fail(DSA_ERR_INVALID_ARG, "cache_insert: tok_req / tok_pos null");
  if (a->block_table && a->bt_stride < 1) return fail(DSA_ERR_INVALID_ARG, "cache_insert: bt_stride < 1");
  dsa::InsertParams p{};
  p.n = a->num_tokens;
  p.R = a->num_requests;
  p.tok_req = a->tok_req;
  p.tok_pos = a->tok_pos;
  p.block_table = a->block_table;
  p.bt_stride = a->bt_stride;
  p.key_vals = static_cast<const uint16_t*>(a->key_vals);
  p.keys = static_cast<uint8_t*>(const_cast<void*>(a->keys.base));  // written by this call
  p.key_page_bytes = a->keys.page_bytes;
  p.key_plog2 = a->keys.page_size_log2;
  p.key_num_pages = a->keys.num_pages;
  p.key_fmt = a->keys.fmt;
  p.lat_vals = static_cast<const uint16_t*>(a->lat_vals);
  p.lat = static_cast<uint8_t*>(const_cast<void*>(a->latents.base));
  p.lat_page_bytes = a->latents.page_bytes;
  p.lat_plog2 = a->latents.page_size_log2;
  p.lat_num_pages = a->latents.num_pages;
  p.lat_fmt = a->latents.fmt;
  const dsa_status st = dsa::launch_cache_insert(p, stream);
  if (st != DSA_OK) return fail(st, "cache_insert: launch failed: %s", hipGetErrorString(hipGetLastError()));
  return DSA_OK;
}

size_t dsa_workspace_size(int32_t op, const void* args) {
  if (!args) return 0;
  switch (op) {
    case DSA_OP_INDEXER: return 0;
    case DSA_OP_TOPK: {
      const dsa_topk_args* a = static_cast<const dsa_topk_args*>(args);
      if (a->k < 1 || a->k > DSA_MAX_TOPK || a->batch.num_rows < 1 || a->batch.max_vis < 1) return 0;
      return plan_topk(a->batch.num_rows, a->batch.max_vis, a->k).total;
    }
    case DSA_OP_INDEXER_PREFIX: {
      const dsa_indexer_prefix_args* a = static_cast<const dsa_indexer_prefix_args*>(args);
      if (a->base.batch.num_rows < 1 || a->num_groups < 1 || a->base.keys.page_size_log2 < 4 ||
          a->base.keys.page_size_log2 > 24 || a->prefix_len < 0)
        return 0;
      return plan_prefix(*a).total;
    }
    case DSA_OP_MSA_DECODE: {
      const dsa_msa_args* a = static_cast<const dsa_msa_args*>(args);
      if (a->batch.num_rows < 1 || a->batch.max_vis < 1 || a->num_kv_heads < 1 || a->num_kv_heads > 8) return 0;
      return align_up((size_t)a->batch.num_rows * a->num_kv_heads * ((a->batch.max_vis + 127) / 128) * 4, 256) +
             align_up((size_t)a->batch.num_rows * a->num_kv_heads * dsa::kMsaSplits * dsa::kMsaPartFloats * 4, 256);
    }
    case DSA_OP_TOPK_SHARDED: {
      const dsa_topk_sharded_args* a = static_cast<const dsa_topk_sharded_args*>(args);
      if (!sharded_shape_ok(*a)) return 0;
      return plan_sharded(*a).total;
    }
    case DSA_OP_MLA_DECODE:
    case DSA_OP_MLA_PREFILL: {
      const dsa_mla_args* a = static_cast<const dsa_mla_args*>(args);
      if (a->k < 1 || a->k > DSA_MAX_TOPK || a->num_rows < 1 || a->num_heads < 1 || a->num_splits < 0) return 0;
      return plan_mla(*a, op == DSA_OP_MLA_PREFILL).total;
    }
  }
  return 0;
}

}  // extern "C"
