// Host-only stand-ins for the library's kernel launchers and for the few HIP
// runtime calls the host ABI makes, so that api.cpp can be built and run on
// the CPU under AddressSanitizer and UndefinedBehaviorSanitizer.
//
// Every "device" buffer the test driver passes is host memory of exactly the
// size the public header documents (workspaces of exactly what
// dsa_workspace_size reports).  Each stub touches the whole extent its kernels
// read or write -- the block table rows the host bound promises, the
// workspace regions the host plan carved out, every output row -- so a host
// plan or check that lets a kernel run past a buffer becomes a sanitizer
// report here rather than a device fault.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "../../include/dsa.h"
#include "../../sparse_attention_03_amd/csrc/kernels.h"

namespace {
volatile uint32_t g_sink;
int g_launches = 0;

// read every byte of [p, p + n)
void read_all(const void* p, size_t n) {
  const volatile uint8_t* b = static_cast<const volatile uint8_t*>(p);
  uint32_t s = 0;
  for (size_t i = 0; i < n; ++i) s += b[i];
  g_sink = g_sink + s;
}
// write every byte of [p, p + n)
void write_all(void* p, size_t n) { std::memset(p, 0x5a, n); }

void need(bool ok, const char* what) {
  if (!ok) {
    std::fprintf(stderr, "launch stub: %s\n", what);
    std::abort();
  }
}

// The rows of a batch-shaped launch: tok_vis and tok_req of every row, the
// request bounds, and the block-table entries a row of max_vis keys names.
void touch_batch(int R, int T, const int32_t* rs, const int32_t* tok_req, const int32_t* tok_vis,
                 const int32_t* bt, int bt_stride, int max_vis, int plog2) {
  need(R >= 1 && T >= 1 && max_vis >= 1, "empty batch reached a launcher");
  read_all(tok_vis, (size_t)T * 4);
  if (tok_req) read_all(tok_req, (size_t)T * 4);
  if (rs) read_all(rs, (size_t)(R + 1) * 4);
  if (bt) {
    const int pages = (int)(((int64_t)max_vis + (1 << plog2) - 1) >> plog2);
    need(bt_stride >= pages, "block table row shorter than max_vis needs");
    for (int r = 0; r < R; ++r) read_all(bt + (int64_t)r * bt_stride, (size_t)pages * 4);
  }
}
}  // namespace

extern "C" int dsa_stub_launches(void) { return g_launches; }

extern "C" {
hipError_t hipGetLastError(void) { return hipSuccess; }
const char* hipGetErrorString(hipError_t) { return "stub"; }
hipError_t hipDeviceSynchronize(void) { return hipSuccess; }
}

namespace dsa {

dsa_status launch_indexer_bf16(const IndexerParams& p, hipStream_t) {
  ++g_launches;
  touch_batch(p.R, p.T, p.req_row_start, p.tok_req, p.tok_vis, p.block_table, p.bt_stride, p.max_vis, p.plog2);
  need(p.ld >= p.max_vis && p.chunk >= 256, "indexer: ld or chunk");
  const size_t qbytes = p.q_e8m0 ? 32 * 64 : 32 * 128 * 2;
  read_all(p.q_e8m0 ? (const void*)p.q8 : (const void*)p.q, (size_t)p.T * qbytes);
  if (p.q_e8m0) read_all(p.q_e8m0, (size_t)p.T * 32 * 4);
  read_all(p.w, (size_t)p.T * 32 * 4);
  write_all(p.scores, ((size_t)(p.T - 1) * p.ld + p.max_vis) * 4);
  read_all(p.keys, (size_t)p.page_bytes * p.num_pages);
  return DSA_OK;
}

dsa_status launch_indexer_fp8(const IndexerParams& p, hipStream_t) {
  ++g_launches;
  touch_batch(p.R, p.T, p.req_row_start, p.tok_req, p.tok_vis, p.block_table, p.bt_stride, p.max_vis, p.plog2);
  read_all(p.q8, (size_t)p.T * 32 * 128);
  read_all(p.q_scale, (size_t)p.T * 32 * 4);
  read_all(p.w, (size_t)p.T * 32 * 4);
  write_all(p.scores, ((size_t)(p.T - 1) * p.ld + p.max_vis) * 4);
  return DSA_OK;
}

dsa_status launch_prefix_prep(const int32_t* tok_vis, int T, int, int, const int32_t* bt, int bt_stride, int R,
                              const int32_t* grs, const int32_t* first_req, int G, int ns_max, int npfx,
                              int32_t* sub_start, int32_t* sub_src, int32_t* vis1, int32_t* vis2, int32_t* ptab,
                              hipStream_t) {
  ++g_launches;
  read_all(tok_vis, (size_t)T * 4);
  read_all(grs, (size_t)(G + 1) * 4);
  read_all(first_req, (size_t)G * 4);
  for (int r = 0; r < R; ++r) read_all(bt + (int64_t)r * bt_stride, (size_t)npfx * 4);
  write_all(sub_start, (size_t)(ns_max + 1) * 4);
  write_all(sub_src, (size_t)ns_max * 4);
  write_all(vis1, (size_t)T * 4);
  write_all(vis2, (size_t)T * 4);
  write_all(ptab, (size_t)ns_max * std::max(1, npfx) * 4);
  // the shared pass then runs with these as its batch: give it a valid one
  for (int i = 0; i <= ns_max; ++i) sub_start[i] = std::min(i, T);
  for (int i = 0; i < T; ++i) vis1[i] = vis2[i] = 1;
  for (int i = 0; i < ns_max * std::max(1, npfx); ++i) ptab[i] = 0;
  return DSA_OK;
}

dsa_status launch_topk(const TopkParams& p, hipStream_t) {
  ++g_launches;
  need(p.T >= 1 && p.k >= 1 && p.k <= DSA_MAX_TOPK, "topk shape");
  read_all(p.tok_vis, (size_t)p.T * 4);
  if (p.tok_req) read_all(p.tok_req, (size_t)p.T * 4);
  read_all(p.scores, ((size_t)(p.T - 1) * p.ld + p.max_vis) * 4);
  write_all(p.idx, (size_t)p.T * p.k * 4);
  if (p.rows) {
    write_all(p.rows, (size_t)p.T * p.k * 4);
    if (p.block_table) {
      need(p.R >= 1, "topk translation without requests");
      for (int r = 0; r < p.R; ++r) read_all(p.block_table + (int64_t)r * p.bt_stride, (size_t)p.bt_stride * 4);
    }
  }
  if (p.count) write_all(p.count, (size_t)p.T * 4);
  write_all(p.ctr, (size_t)p.T * 16);
  write_all(p.cand, (size_t)p.T * p.nslices * p.slice_cap * 8);
  need(p.slice_cap >= 1 && p.slice_cap <= p.cand_cap, "topk slice region");
  write_all(p.slice_info, (size_t)p.T * p.nslices * 8);
  need(p.cand_cap >= std::min(p.max_vis, kTopkFinalCap), "topk candidate buffer");
  need((int64_t)p.nslices * p.slice >= p.max_vis, "topk slices");
  return DSA_OK;
}

dsa_status launch_topk_sharded(const MergeParams& m, const TopkParams& local, hipStream_t s) {
  ++g_launches;
  const size_t n = (size_t)m.W * m.T;
  read_all(m.tok_vis, (size_t)m.T * 4);
  write_all(m.idx, (size_t)m.T * m.k * 4);
  if (m.count) write_all(m.count, (size_t)m.T * 4);
  write_all(m.lvis, n * 4);
  write_all(m.lvis2, n * 4);
  write_all(m.lidx, n * std::max(m.k, m.cand) * 4);
  write_all(m.xbuf, n * m.k * 8);
  write_all(m.xcnt, n * 4);
  write_all(m.flags, (size_t)m.T * m.W * 4);
  write_all(m.rowflag, (size_t)m.T * 4);
  need(local.idx == m.lidx && (size_t)local.T == n, "sharded local top-k shape");
  for (size_t i = 0; i < n; ++i) m.lvis[i] = 1;  // the local pass reads them as its visible counts
  return launch_topk(local, s);
}

dsa_status launch_translate(const int32_t* idx, int k, int T, const int32_t* tok_req, int R, const int32_t* bt,
                            int bt_stride, int, int, int32_t* rows, hipStream_t) {
  ++g_launches;
  need(R >= 1, "translate without requests");
  read_all(idx, (size_t)T * k * 4);
  read_all(tok_req, (size_t)T * 4);
  if (bt)
    for (int r = 0; r < R; ++r) read_all(bt + (int64_t)r * bt_stride, (size_t)bt_stride * 4);
  write_all(rows, (size_t)T * k * 4);
  return DSA_OK;
}

dsa_status launch_mla(const MlaParams& p, hipStream_t) {
  ++g_launches;
  need(p.T >= 1 && p.H >= 1 && p.Hpad >= p.H && p.Hpad % 16 == 0 && p.ntiles * 16 == p.Hpad, "mla heads");
  need(p.nsplit >= 1 && (int64_t)p.nsplit * p.split_len >= p.k && p.split_len % 16 == 0, "mla split plan");
  read_all(p.q, (size_t)p.T * p.H * 576 * 2);
  read_all(p.rows, (size_t)p.T * p.k * 4);
  write_all(p.out, (size_t)p.T * p.H * 512 * 4);
  if (p.lse) write_all(p.lse, (size_t)p.T * p.H * 4);
  if (p.nsplit > 1) {
    write_all(p.part_o, (size_t)p.T * p.nsplit * p.H * 512 * 4);
    write_all(p.part_lse, (size_t)p.T * p.nsplit * p.H * 4);
  }
  return DSA_OK;
}

dsa_status mla_scratch(void** ptr) {
  static void* s = nullptr;
  if (!s) s = std::malloc(kMlaScratchBytes);
  *ptr = s;
  return s ? DSA_OK : DSA_ERR_HIP;
}

dsa_status launch_quantize_q(const QuantQParams& p, hipStream_t) {
  ++g_launches;
  read_all(p.q, (size_t)p.T * 32 * 128 * 2);
  if (p.fmt == DSA_Q_FP8) {
    write_all(p.out, (size_t)p.T * 32 * 128);
    write_all(p.scale, (size_t)p.T * 32 * 4);
    if (p.w_folded) {
      read_all(p.w, (size_t)p.T * 32 * 4);
      write_all(p.w_folded, (size_t)p.T * 32 * 4);
    }
  } else {
    write_all(p.out, (size_t)p.T * 32 * 64);
    write_all(p.scale, (size_t)p.T * 32 * 4);
  }
  return DSA_OK;
}

dsa_status launch_cache_insert(const InsertParams& p, hipStream_t) {
  ++g_launches;
  read_all(p.tok_req, (size_t)p.n * 4);
  read_all(p.tok_pos, (size_t)p.n * 4);
  if (p.key_vals) read_all(p.key_vals, (size_t)p.n * 128 * 2);
  if (p.lat_vals) read_all(p.lat_vals, (size_t)p.n * 576 * 2);
  if (p.keys) write_all(p.keys, (size_t)p.key_page_bytes * p.key_num_pages);
  if (p.lat) write_all(p.lat, (size_t)p.lat_page_bytes * p.lat_num_pages);
  return DSA_OK;
}

dsa_status launch_msa(const MsaParams& p, int nblk_max, hipStream_t) {
  ++g_launches;
  touch_batch(p.R, p.T, p.req_row_start, p.tok_req, p.tok_vis, p.bt, p.bt_stride, p.max_vis, 7);
  need(p.nblk_ld >= nblk_max && nblk_max * 128 >= p.max_vis, "msa block scores");
  read_all(p.q_idx, (size_t)p.T * p.hkv * 128 * 2);
  read_all(p.q, (size_t)p.T * p.hq * 128 * 2);
  write_all(p.bscore, (size_t)p.T * p.hkv * p.nblk_ld * 4);
  write_all(p.part, (size_t)p.T * p.hkv * kMsaSplits * kMsaPartFloats * 4);
  write_all(p.sel, (size_t)p.T * p.hkv * p.top * 4);
  write_all(p.out, (size_t)p.T * p.hq * 128 * 4);
  if (p.lse) write_all(p.lse, (size_t)p.T * p.hq * 4);
  read_all(p.idx_pool, (size_t)p.pool_blocks * 128 * 128);
  read_all(p.kv_pool, (size_t)p.pool_blocks * 128 * 2 * p.hkv * 128);
  return DSA_OK;
}

uint32_t debug_take_indexer() { return 0; }
uint32_t debug_take_indexer_fp8() { return 0; }
uint32_t debug_take_topk() { return 0; }
uint32_t debug_take_mla() { return 0; }
uint32_t debug_take_quant() { return 0; }
uint32_t debug_take_merge() { return 0; }
uint32_t debug_take_msa() { return 0; }

}  // namespace dsa
