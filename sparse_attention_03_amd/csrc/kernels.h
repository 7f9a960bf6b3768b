// Kernel parameter blocks and launchers (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/dsa.h"

namespace dsa {

// Query rows of a request the BF16 indexer stages in LDS per pass.
constexpr int kIndexerMaxRowsPerPass = 6;
// FP8 queries of requests with at most this many rows run on the multi-row
// decode kernel (FP8 instruction, raw keys); more rows per request on the
// prefill kernel
constexpr int kIndexerQ8MaxRows = 8;
// Keys per workgroup of the single-row BF16 indexer (its LDS holds the
// chunk's scores): FP8 keys, MXFP4 / NVFP4 keys.
constexpr int kIndexerRowChunkFp8 = 2048;
constexpr int kIndexerRowChunkFp4 = 4096;

struct IndexerParams {
  int R, T;
  const int32_t* req_row_start;
  const int32_t* tok_req;
  const int32_t* tok_vis;
  const int32_t* block_table;
  int bt_stride;
  int max_vis;
  // key pool
  const uint8_t* keys;
  int64_t page_bytes;
  int plog2;
  int num_pages;
  int key_fmt;
  // queries
  const __bf16* q;          // bf16 q (BF16 path)
  const uint8_t* q8;        // E4M3 q (FP8 path), E2M1 pairs (MXFP4 path)
  const float* q_scale;     // [T,32] (FP8 path)
  const uint8_t* q_e8m0;    // [T,32,4] (MXFP4 path)
  const float* w;           // [T,32]
  float* scores;
  int64_t ld;
  int chunk;                // keys per workgroup (a multiple of 256)
  int qrows;                // rows staged in LDS per pass (BF16 path)
  int max_rows_per_req;
};

// Candidates per row the top-k finalize holds in LDS (the candidate buffer
// holds at most this many per row).
constexpr int kTopkFinalCap = 8192;

struct TopkParams {
  int T;
  const float* scores;
  int64_t ld;
  const int32_t* tok_vis;
  const int32_t* tok_req;
  int R;                // requests: a row whose tok_req is outside [0, R) translates to -1
  int max_vis;
  int k;
  const int32_t* block_table;
  int bt_stride;
  int plog2;
  int num_pages;        // latent pool pages: translation maps other pages to -1
  int32_t* idx;
  int32_t* rows;
  int32_t* count;
  // workspace
  uint32_t* ctr;        // [T][4]: -, -, threshold key, -
  uint32_t* cand;       // [T][nslices][slice_cap][2]: each slice's candidates (order key, index)
  uint32_t* slice_info; // [T][nslices][2]: -, count of each slice's candidates
  int cand_cap;         // candidates the finalize selects from in LDS
  int slice_cap;        // candidate entries of one slice's region
  int slice;            // scores per workgroup in the filter pass
  int nslices;
  int skip_empty;       // rows with no visible score write nothing (not even padding)
};

// Shards of the sharded top-k merge (context shards of one row).
constexpr int kMaxShards = 16;

struct MergeParams {
  int T, W, k, cand;
  const float* scores;  // [W][T][ld] shard-local scores
  int64_t ld;
  const int32_t* tok_vis;
  int max_vis;
  int32_t* idx;         // [T][k]
  int32_t* count;       // [T] or null
  // workspace
  int32_t* lvis;        // [W*T] local visible counts (shard row r*T + t)
  int32_t* lvis2;       // [W*T] re-send local counts: lvis for flagged shard rows, else 0
  int32_t* lidx;        // [W*T][cand] then [W*T][k]: selected local positions
  uint64_t* xbuf;       // [W*T][k] exchange buffer: composites each shard row sent
  int32_t* xcnt;        // [W*T] composites sent
  int32_t* flags;       // [T][W] re-send flags
  int32_t* rowflag;     // [T] any re-send in the row
};

struct MlaParams {
  int T, H, Hpad, ntiles;
  const __bf16* q;
  const uint8_t* lat;
  int64_t page_bytes;
  int plog2;
  int num_pages;
  int fmt;
  const int32_t* rows;
  int k;
  float sm_log2;            // sm_scale * log2(e)
  int nsplit;
  int split_len;            // list entries per split (multiple of 16)
  float* out;
  float* lse;
  float* part_o;            // [T][nsplit][H][512]
  float* part_lse;          // [T][nsplit][H]
  int prefill;              // one split per row over all heads (sparse_mla_prefill)
};

// Workgroup shape of the sparse-MLA kernels: `groups` workgroups per (row,
// split), each with nw / vs head tiles of 16 heads; a workgroup's LDS tile
// takes a quarter of a CU's LDS per head tile it serves, so 4 / (nw / vs)
// workgroups share a CU.
struct MlaShape {
  int groups, nw, vs, resident_per_cu;
};
// vs waves per head tile, each holding 512 / vs of the value dims: two when
// the heads fill a single tile and the latents are NVFP4 (whose dequantisation
// the two waves then share; both compute the tile's scores, each multiplies
// its half of the values).  For FP8 latents the second wave only repeats the
// score chain that bounds the tile, so it stays at one.
// Prefill over FP8 latents (the ring kernel, about 20 KB of LDS per workgroup
// whatever its waves): one wave per head tile, eight waves per CU (two per
// SIMD, the register limit) -- one workgroup for up to two head tiles, else
// workgroups of two (96 heads: three per row) or four.
inline MlaShape mla_shape_fp8(int ntiles) {
  MlaShape s;
  s.nw = ntiles <= 2 ? ntiles : (ntiles % 4 == 0 ? 4 : 2);
  s.groups = (ntiles + s.nw - 1) / s.nw;
  s.vs = 1;
  s.resident_per_cu = 8 / s.nw;
  return s;
}
inline MlaShape mla_shape(int ntiles, bool split_values) {
  MlaShape s;
  s.groups = (ntiles + 3) / 4;
  const int tiles = (ntiles + s.groups - 1) / s.groups;
  s.vs = (split_values && ntiles == 1) ? 2 : 1;
  s.nw = tiles * s.vs;
  s.resident_per_cu = 4 / tiles;
  return s;
}

struct QuantQParams {
  int T;
  const uint16_t* q;   // bf16 bits [T][32][128]
  const float* w;
  int fmt;             // DSA_Q_FP8 or DSA_Q_MXFP4
  uint8_t* out;
  void* scale;
  float* w_folded;
};

struct InsertParams {
  int n, R;
  const int32_t* tok_req;
  const int32_t* tok_pos;
  const int32_t* block_table;
  int bt_stride;
  const uint16_t* key_vals;  // bf16 bits [n][128] or null
  uint8_t* keys;
  int64_t key_page_bytes;
  int key_plog2, key_num_pages, key_fmt;
  const uint16_t* lat_vals;  // bf16 bits [n][576] or null
  uint8_t* lat;
  int64_t lat_page_bytes;
  int lat_plog2, lat_num_pages, lat_fmt;
};

dsa_status launch_quantize_q(const QuantQParams& p, hipStream_t stream);
dsa_status launch_cache_insert(const InsertParams& p, hipStream_t stream);
dsa_status launch_indexer_bf16(const IndexerParams& p, hipStream_t stream);
dsa_status launch_indexer_fp8(const IndexerParams& p, hipStream_t stream);
// Attention workgroups per (row, group) of the MSA decode, and the floats of
// one workgroup's partial result (16 maxima, 16 sums, 16 x 128 outputs).
constexpr int kMsaSplits = 2;
constexpr int kMsaPartFloats = 16 * 128 + 32;

struct MsaParams {
  int R, T, hkv, hq, G, top, nblk_ld;
  const int32_t* req_row_start;
  const int32_t* tok_req;
  const int32_t* tok_vis;
  int max_vis;
  const int32_t* bt;
  int bt_stride;
  int pool_blocks;
  const uint8_t* idx_pool;  // [blocks][128 tokens][128] E4M3
  const uint8_t* kv_pool;   // [blocks][128 tokens][2][hkv][128] E4M3
  const __bf16* q_idx;      // [T][hkv][128]
  const __bf16* q;          // [T][hq][128]
  float k_scale, v_scale, sm_scale;
  float* bscore;            // workspace [T][hkv][nblk_ld]
  float* part;              // workspace [T*hkv][kMsaSplits][kMsaPartFloats]
  int32_t* sel;             // [T][hkv][top]
  float* out;               // [T][hq][128]
  float* lse;               // [T][hq] or null
};

dsa_status launch_topk(const TopkParams& p, hipStream_t stream);
dsa_status launch_msa(const MsaParams& p, int nblk_max, hipStream_t stream);
// Rows of one shared-prefix pass (two of the multi-row indexer's row passes:
// measured fastest on 64 single-row requests sharing 192K of 256K tokens).
constexpr int kPrefixSubRows = 12;
dsa_status launch_prefix_prep(const int32_t* tok_vis, int T, int max_vis, int L, const int32_t* bt, int bt_stride,
                              int R, const int32_t* grs, const int32_t* first_req, int G, int ns_max, int npfx,
                              int32_t* sub_start, int32_t* sub_src, int32_t* vis1, int32_t* vis2, int32_t* ptab,
                              hipStream_t stream);
dsa_status launch_topk_sharded(const MergeParams& p, const TopkParams& local, hipStream_t stream);
dsa_status launch_translate(const int32_t* idx, int k, int T, const int32_t* tok_req, int R,
                            const int32_t* block_table, int bt_stride, int plog2, int num_pages, int32_t* rows,
                            hipStream_t stream);
dsa_status launch_mla(const MlaParams& p, hipStream_t stream);
// Bytes of the device-resident scratch of sparse_mla_decode_noalloc (split
// partials), and its address on the current device (resolved on first use).
constexpr size_t kMlaScratchBytes = DSA_MLA_SCRATCH_BYTES;
dsa_status mla_scratch(void** ptr);

// Debug notes of each source file (dsa_check_debug_flag): the bits noted
// since the last call, cleared; always 0 in release builds.
uint32_t debug_take_indexer();
uint32_t debug_take_indexer_fp8();
uint32_t debug_take_topk();
uint32_t debug_take_mla();
uint32_t debug_take_quant();
uint32_t debug_take_merge();
uint32_t debug_take_msa();

}  // namespace dsa
