// Drives every entry point of the host ABI (api.cpp) on the CPU, linked with
// launch_stubs.cpp, under AddressSanitizer and UndefinedBehaviorSanitizer:
// valid calls on decode, speculative, prefill, sharded, MSA and shared-prefix
// shapes with buffers of exactly their documented sizes (workspaces of
// exactly dsa_workspace_size), then argument errors that must be rejected
// before any launch.  Prints "abi driver ok: N calls, M launches" on success;
// any failed expectation or sanitizer report ends the process non-zero.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../../include/dsa.h"

extern "C" int dsa_stub_launches(void);

namespace {

int g_calls = 0;
std::vector<void*> g_bufs;

// host memory standing in for a device buffer of exactly `bytes`
template <class T = void>
T* buf(size_t bytes, size_t align = 256) {
  void* p = nullptr;
  if (posix_memalign(&p, align, bytes ? bytes : 1) != 0) std::abort();
  std::memset(p, 0, bytes ? bytes : 1);
  g_bufs.push_back(p);
  return static_cast<T*>(p);
}

void expect(dsa_status got, dsa_status want, const char* what) {
  ++g_calls;
  if (got != want) {
    std::fprintf(stderr, "%s: got %s, expected %s (%s)\n", what, dsa_status_str(got), dsa_status_str(want),
                 dsa_last_error());
    std::exit(1);
  }
}

// A batch of R requests with `rows` rows each, paged with page size 2^plog2.
struct Batch {
  dsa_batch b;
  int32_t *rs, *req, *vis, *bt;
};
Batch make_batch(int R, int rows, int max_vis, int plog2, bool paged = true) {
  Batch x{};
  const int T = R * rows;
  const int pages = (max_vis + (1 << plog2) - 1) >> plog2;
  x.rs = buf<int32_t>((size_t)(R + 1) * 4);
  x.req = buf<int32_t>((size_t)T * 4);
  x.vis = buf<int32_t>((size_t)T * 4);
  for (int r = 0; r <= R; ++r) x.rs[r] = r * rows;
  for (int t = 0; t < T; ++t) {
    x.req[t] = t / rows;
    x.vis[t] = max_vis - (rows - 1 - t % rows);
  }
  x.bt = nullptr;
  if (paged) {
    x.bt = buf<int32_t>((size_t)R * pages * 4);
    for (int i = 0; i < R * pages; ++i) x.bt[i] = i;
  }
  x.b = dsa_batch{R, T, x.rs, x.req, x.vis, x.bt, paged ? pages : 0, max_vis, rows};
  return x;
}

dsa_cache key_pool(int fmt, int plog2, int pages) {
  const int tb = fmt == DSA_KEY_FP8 ? 132 : fmt == DSA_KEY_MXFP4 ? 68 : 72;
  const int64_t pb = (int64_t)tb << plog2;
  return dsa_cache{buf((size_t)pb * pages), pb, plog2, pages, fmt};
}
dsa_cache lat_pool(int fmt, int plog2, int pages) {
  const int rb = fmt == DSA_LAT_BF16 ? 1152 : fmt == DSA_LAT_FP8 ? 640 : 384;
  const int64_t pb = (int64_t)rb << plog2;
  return dsa_cache{buf((size_t)pb * pages), pb, plog2, pages, fmt};
}

void indexer_case(int R, int rows, int max_vis, int plog2, int kfmt, int qfmt) {
  Batch x = make_batch(R, rows, max_vis, plog2);
  const int T = R * rows;
  const int64_t ld = (max_vis + 3) / 4 * 4;
  dsa_indexer_args a{};
  a.batch = x.b;
  a.keys = key_pool(kfmt, plog2, R * x.b.bt_stride);
  a.q_fmt = qfmt;
  a.q = buf((size_t)T * 32 * (qfmt == DSA_Q_BF16 ? 256 : qfmt == DSA_Q_FP8 ? 128 : 64));
  a.q_scale = qfmt == DSA_Q_BF16 ? nullptr : buf((size_t)T * 32 * 4);
  a.w = buf<float>((size_t)T * 32 * 4);
  a.scores = buf<float>((size_t)T * ld * 4);
  a.ld = ld;
  expect(dsa_indexer_scores(&a, nullptr), DSA_OK, "indexer");
  // errors: ld below max_vis, a block table too short for max_vis, unaligned q
  dsa_indexer_args e = a;
  e.ld = ld - 4;
  expect(dsa_indexer_scores(&e, nullptr), DSA_ERR_INVALID_ARG, "indexer ld");
  e = a;
  e.batch.bt_stride -= 1;
  expect(dsa_indexer_scores(&e, nullptr), DSA_ERR_INVALID_ARG, "indexer bt_stride");
  e = a;
  e.q = static_cast<const char*>(a.q) + 4;
  expect(dsa_indexer_scores(&e, nullptr), DSA_ERR_INVALID_ARG, "indexer q alignment");
}

void topk_case(int R, int rows, int max_vis, int k, int plog2) {
  Batch x = make_batch(R, rows, max_vis, plog2);
  const int T = R * rows;
  dsa_topk_args a{};
  a.batch = x.b;
  a.ld = (max_vis + 3) / 4 * 4;
  a.scores = buf<float>((size_t)T * a.ld * 4);
  a.k = k;
  a.idx = buf<int32_t>((size_t)T * k * 4);
  a.rows = buf<int32_t>((size_t)T * k * 4);
  a.count = buf<int32_t>((size_t)T * 4);
  a.page_size_log2 = plog2;
  a.num_pages = R * x.b.bt_stride;
  const size_t ws = dsa_workspace_size(DSA_OP_TOPK, &a);
  a.workspace = buf(ws);
  a.workspace_bytes = ws;
  expect(dsa_topk(&a, nullptr), DSA_OK, "topk");
  dsa_topk_args e = a;
  e.workspace_bytes = ws - 1;
  expect(dsa_topk(&e, nullptr), DSA_ERR_WORKSPACE, "topk workspace");
  e = a;
  e.k = DSA_MAX_TOPK + 1;
  expect(dsa_topk(&e, nullptr), DSA_ERR_INVALID_ARG, "topk k");
  e = a;
  e.num_pages = 0;
  expect(dsa_topk(&e, nullptr), DSA_ERR_INVALID_ARG, "topk num_pages");
  expect(dsa_translate_pages(a.idx, k, &a.batch, plog2, a.num_pages, a.rows, nullptr), DSA_OK, "translate");
  expect(dsa_translate_pages(a.idx, 0, &a.batch, plog2, a.num_pages, a.rows, nullptr), DSA_ERR_INVALID_ARG,
         "translate k");
}

void mla_case(int T, int H, int k, int lfmt, int splits, bool prefill) {
  dsa_mla_args a{};
  a.num_rows = T;
  a.num_heads = H;
  a.q = buf((size_t)T * H * 576 * 2);
  a.latents = lat_pool(lfmt, 6, 64);
  a.rows = buf<int32_t>((size_t)T * k * 4);
  a.k = k;
  a.sm_scale = 0.0721f;
  a.num_splits = splits;
  a.out = buf<float>((size_t)T * H * 512 * 4);
  a.lse = buf<float>((size_t)T * H * 4);
  const size_t ws = dsa_workspace_size(prefill ? DSA_OP_MLA_PREFILL : DSA_OP_MLA_DECODE, &a);
  a.workspace = ws ? buf(ws) : nullptr;
  a.workspace_bytes = ws;
  expect(prefill ? sparse_mla_prefill(&a, nullptr) : sparse_mla_decode(&a, nullptr), DSA_OK, "mla");
  if (!prefill) {
    expect(sparse_mla_decode_noalloc(&a, nullptr), DSA_OK, "mla noalloc");
    if (ws) {
      dsa_mla_args e = a;
      e.workspace_bytes = ws - 1;
      expect(sparse_mla_decode(&e, nullptr), DSA_ERR_WORKSPACE, "mla workspace");
    }
  }
  dsa_mla_args e = a;
  e.num_heads = DSA_MAX_HEADS + 1;
  expect(sparse_mla_decode(&e, nullptr), DSA_ERR_INVALID_ARG, "mla heads");
  e = a;
  e.sm_scale = 0.f;
  expect(sparse_mla_decode(&e, nullptr), DSA_ERR_INVALID_ARG, "mla sm_scale");
}

void sharded_case(int T, int W, int max_vis, int k) {
  dsa_topk_sharded_args a{};
  a.num_rows = T;
  a.num_shards = W;
  a.ld = ((max_vis + W - 1) / W + 3) / 4 * 4;
  a.scores = buf<float>((size_t)W * T * a.ld * 4);
  a.tok_vis = buf<int32_t>((size_t)T * 4);
  a.max_vis = max_vis;
  a.k = k;
  a.idx = buf<int32_t>((size_t)T * k * 4);
  a.count = buf<int32_t>((size_t)T * 4);
  a.resend = buf<int32_t>((size_t)T * W * 4);
  const size_t ws = dsa_workspace_size(DSA_OP_TOPK_SHARDED, &a);
  a.workspace = buf(ws);
  a.workspace_bytes = ws;
  expect(dsa_topk_sharded(&a, nullptr), DSA_OK, "topk_sharded");
  dsa_topk_sharded_args e = a;
  e.num_shards = 17;
  expect(dsa_topk_sharded(&e, nullptr), DSA_ERR_INVALID_ARG, "topk_sharded W");
  e = a;
  e.workspace_bytes = ws - 1;
  expect(dsa_topk_sharded(&e, nullptr), DSA_ERR_WORKSPACE, "topk_sharded workspace");
}

void msa_case(int R, int max_vis, int hkv, int hq, int top) {
  Batch x = make_batch(R, 1, max_vis, 7);
  const int T = R;
  const int blocks = R * x.b.bt_stride;
  dsa_msa_args a{};
  a.batch = x.b;
  a.index_keys = buf((size_t)blocks * 128 * 128);
  a.kv = buf((size_t)blocks * 128 * 2 * hkv * 128);
  a.num_blocks = blocks;
  a.num_kv_heads = hkv;
  a.num_q_heads = hq;
  a.top_blocks = top;
  a.q_idx = buf((size_t)T * hkv * 128 * 2);
  a.q = buf((size_t)T * hq * 128 * 2);
  a.k_scale = a.v_scale = 1.f;
  a.sm_scale = 0.088f;
  a.sel_blocks = buf<int32_t>((size_t)T * hkv * top * 4);
  a.out = buf<float>((size_t)T * hq * 128 * 4);
  a.lse = buf<float>((size_t)T * hq * 4);
  const size_t ws = dsa_workspace_size(DSA_OP_MSA_DECODE, &a);
  a.workspace = buf(ws);
  a.workspace_bytes = ws;
  expect(dsa_msa_decode(&a, nullptr), DSA_OK, "msa");
  dsa_msa_args e = a;
  e.num_q_heads = hkv * 17;
  expect(dsa_msa_decode(&e, nullptr), DSA_ERR_INVALID_ARG, "msa heads");
  e = a;
  e.workspace_bytes = ws - 1;
  expect(dsa_msa_decode(&e, nullptr), DSA_ERR_WORKSPACE, "msa workspace");
}

void prefix_case(int groups, int per_group, int max_vis, int prefix, int plog2) {
  const int R = groups * per_group;
  Batch x = make_batch(R, 1, max_vis, plog2);
  dsa_indexer_prefix_args a{};
  dsa_indexer_args& b = a.base;
  b.batch = x.b;
  b.keys = key_pool(DSA_KEY_FP8, plog2, R * x.b.bt_stride);
  b.q_fmt = DSA_Q_BF16;
  b.q = buf((size_t)R * 32 * 256);
  b.w = buf<float>((size_t)R * 32 * 4);
  b.ld = (max_vis + 3) / 4 * 4;
  b.scores = buf<float>((size_t)R * b.ld * 4);
  int32_t* grs = buf<int32_t>((size_t)(groups + 1) * 4);
  int32_t* first = buf<int32_t>((size_t)groups * 4);
  for (int g = 0; g <= groups; ++g) grs[g] = g * per_group;
  for (int g = 0; g < groups; ++g) first[g] = g * per_group;
  a.num_groups = groups;
  a.group_row_start = grs;
  a.group_first_req = first;
  a.prefix_len = prefix;
  a.max_rows_per_group = per_group;
  const size_t ws = dsa_workspace_size(DSA_OP_INDEXER_PREFIX, &a);
  a.workspace = buf(ws);
  a.workspace_bytes = ws;
  expect(dsa_indexer_scores_prefix(&a, nullptr), DSA_OK, "indexer_prefix");
  dsa_indexer_prefix_args e = a;
  e.prefix_len = prefix + 1;
  expect(dsa_indexer_scores_prefix(&e, nullptr), DSA_ERR_INVALID_ARG, "indexer_prefix prefix_len");
}

void front_end_case(int T) {
  dsa_quant_q_args q{};
  q.num_rows = T;
  q.q = buf((size_t)T * 32 * 256);
  q.w = buf<float>((size_t)T * 32 * 4);
  q.fmt = DSA_Q_FP8;
  q.q_out = buf((size_t)T * 32 * 128);
  q.q_scale = buf((size_t)T * 32 * 4);
  q.w_folded = buf<float>((size_t)T * 32 * 4);
  expect(dsa_quantize_q(&q, nullptr), DSA_OK, "quantize fp8");
  dsa_quant_q_args m = q;
  m.fmt = DSA_Q_MXFP4;
  m.w_folded = nullptr;
  m.q_out = buf((size_t)T * 32 * 64);
  m.q_scale = buf((size_t)T * 32 * 4);
  expect(dsa_quantize_q(&m, nullptr), DSA_OK, "quantize mxfp4");
  m.w_folded = q.w_folded;
  expect(dsa_quantize_q(&m, nullptr), DSA_ERR_INVALID_ARG, "quantize mxfp4 with w_folded");

  const int R = 3, pages = 4, plog2 = 6;
  dsa_insert_args in{};
  in.num_tokens = T;
  in.num_requests = R;
  in.tok_req = buf<int32_t>((size_t)T * 4);
  in.tok_pos = buf<int32_t>((size_t)T * 4);
  in.block_table = buf<int32_t>((size_t)R * pages * 4);
  in.bt_stride = pages;
  in.key_vals = buf((size_t)T * 256);
  in.lat_vals = buf((size_t)T * 1152);
  for (int kf : {DSA_KEY_FP8, DSA_KEY_MXFP4, DSA_KEY_NVFP4})
    for (int lf : {DSA_LAT_BF16, DSA_LAT_FP8, DSA_LAT_NVFP4}) {
      in.keys = key_pool(kf, plog2, R * pages);
      in.latents = lat_pool(lf, plog2, R * pages);
      expect(dsa_cache_insert(&in, nullptr), DSA_OK, "cache_insert");
    }
  dsa_insert_args e = in;
  e.latents.page_size_log2 = plog2 + 1;
  expect(dsa_cache_insert(&e, nullptr), DSA_ERR_INVALID_ARG, "cache_insert page sizes");
}

}  // namespace

int main() {
  if (dsa_abi_version() != DSA_ABI_VERSION) return 1;
  // decode (one row per request), speculative verify (rows of one request),
  // the three key formats, FP8 and MXFP4 queries
  indexer_case(8, 1, 20000, 6, DSA_KEY_FP8, DSA_Q_BF16);
  indexer_case(4, 4, 9000, 6, DSA_KEY_MXFP4, DSA_Q_BF16);
  indexer_case(4, 4, 9000, 6, DSA_KEY_NVFP4, DSA_Q_BF16);
  indexer_case(2, 64, 4099, 6, DSA_KEY_FP8, DSA_Q_FP8);
  indexer_case(6, 1, 12345, 6, DSA_KEY_MXFP4, DSA_Q_MXFP4);
  // top-k below and above the candidate buffer's cap, k of 1 and 2048
  topk_case(4, 1, 3000, 2048, 6);
  topk_case(3, 2, 70001, 2048, 6);
  topk_case(2, 1, 5, 1, 4);
  // MLA: padded heads, automatic and explicit splits, every latent format
  mla_case(8, 12, 2048, DSA_LAT_FP8, 0, false);
  mla_case(3, 128, 2048, DSA_LAT_BF16, 0, false);
  mla_case(5, 16, 777, DSA_LAT_NVFP4, 7, false);
  mla_case(4, 96, 2048, DSA_LAT_FP8, 0, true);
  sharded_case(3, 8, 100000, 2048);
  sharded_case(2, 1, 500, 64);
  msa_case(3, 5000, 2, 16, 8);
  prefix_case(2, 3, 4096, 2048, 6);
  prefix_case(1, 2, 1000, 0, 6);
  front_end_case(5);
  // null arguments
  expect(dsa_indexer_scores(nullptr, nullptr), DSA_ERR_INVALID_ARG, "indexer null");
  expect(dsa_topk(nullptr, nullptr), DSA_ERR_INVALID_ARG, "topk null");
  expect(sparse_mla_decode(nullptr, nullptr), DSA_ERR_INVALID_ARG, "mla null");
  expect(sparse_mla_decode_noalloc(nullptr, nullptr), DSA_ERR_INVALID_ARG, "mla noalloc null");
  expect(dsa_msa_decode(nullptr, nullptr), DSA_ERR_INVALID_ARG, "msa null");
  if (dsa_workspace_size(DSA_OP_TOPK, nullptr) != 0) return 1;
  if (dsa_check_debug_flag() != -1) return 1;
  const int launches = dsa_stub_launches();
  for (void* p : g_bufs) std::free(p);
  std::printf("abi driver ok: %d calls, %d launches\n", g_calls, launches);
  return 0;
}
