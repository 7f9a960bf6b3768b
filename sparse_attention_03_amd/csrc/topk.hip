// Per-row top-k with a lower-index tie-break, and block-table translation.
//
// Kimi K3.1 Pro day-0 page: "Sparse attention in K3.1 Pro" keeps the 2,048
// best-scored tokens per query; "Exact top-k merge" selects by radix select;
// AMD "Communication" asks for a consistent tie-break rule.  The set kept for
// row t is unique: the K = min(k, vis) largest scores, equal scores ordered by
// ascending index.  It is emitted in ascending index order.
//
// One pass over the scores, bracketed by two small per-row kernels:
//   1. threshold: one workgroup per row reads a sample of the row -- every
//      score when the row is short, else the first 16 scores (one 64-byte
//      line) of every block of B -- and finds, by two 12-bit histogram
//      levels over the sample's key range, a key tau with about
//      K * S / vis + 4 sqrt(.) + 8 sample keys at or above it (exactly the
//      K-th largest key when the whole row is the sample).  So with
//      overwhelming probability at least K and not many more than K scores
//      of the row are >= tau.
//   2. filter: the row is cut into slices; every slice writes its keys >=
//      tau, in index order, to a region of the candidate buffer of its own
//      (no atomic shared by the row's workgroups) and records their count.
//   3. finalize: one workgroup per row puts the candidates in index order
//      (blocks by slice), runs an exact radix select (12-bit digits) over
//      their 64-bit composites (key, inverted index) -- ties go to the lower
//      index -- and a stable compaction of the winners is the ordered result;
//      it writes indices and physical rows.
// The estimate only decides speed: when fewer than K candidates arrived, more
// than the finalize holds, or more than a slice's region holds, finalize
// selects from the whole score row instead (same result).
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "radix.h"

namespace dsa {

constexpr int kExactMax = 8192;     // rows up to this length are sampled completely
constexpr int kMaxSamples = 16384;  // 16 per thread of the threshold workgroup
constexpr int kRun = 32;            // consecutive scores per sampled block (one 128-byte line)

__device__ __forceinline__ int row_vis(const TopkParams& p, int t) {
  return clamp_vis(p.tok_vis[t], p.max_vis);
}

// Request of row t, or -1 when tok_req names none of the batch's requests
// (its translated rows are then -1: no block-table row is read).
__device__ __forceinline__ int req_or_none(int r, int R) {
  DSA_DEBUG_NOTE(r < 0 || r >= R, DSA_DEBUG_REQ_OUTSIDE);
  return (r >= 0 && r < R) ? r : -1;
}
__device__ __forceinline__ int row_req(const TopkParams& p, int t) {
  return p.tok_req ? req_or_none(p.tok_req[t], p.R) : 0;
}

// Wave-wide scans and reductions on DPP lane moves (no LDS round trip): the
// inclusive prefix sum is radix.h's wave_incl_scan32; maxima take the same
// shifts and row broadcasts; totals are read from lane 63.
__device__ __forceinline__ uint32_t wave_scan_incl(uint32_t v) { return wave_incl_scan32(v); }
__device__ __forceinline__ uint32_t wave_total(uint32_t incl) { return (uint32_t)__builtin_amdgcn_readlane((int)incl, 63); }
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
__device__ __forceinline__ uint32_t wave_min(uint32_t v) { return ~wave_max(~v); }
// 64-bit max: each step moves both halves of the neighbour's value.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  auto step = [&](auto ctrl, int row_mask) {
    (void)ctrl;
    constexpr int c = decltype(ctrl)::value;
    uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32), nl, nh;
    if (row_mask == 0xf) {
      nl = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)lo, c, 0xf, 0xf, false);
      nh = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)hi, c, 0xf, 0xf, false);
    } else if (row_mask == 0xa) {
      nl = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)lo, c, 0xa, 0xf, false);
      nh = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)hi, c, 0xa, 0xf, false);
    } else {
      nl = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)lo, c, 0xc, 0xf, false);
      nh = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)hi, c, 0xc, 0xf, false);
    }
    const uint64_t n = ((uint64_t)nh << 32) | nl;
    v = n > v ? n : v;
  };
  step(std::integral_constant<int, 0x111>{}, 0xf);
  step(std::integral_constant<int, 0x112>{}, 0xf);
  step(std::integral_constant<int, 0x114>{}, 0xf);
  step(std::integral_constant<int, 0x118>{}, 0xf);
  step(std::integral_constant<int, 0x142>{}, 0xa);
  step(std::integral_constant<int, 0x143>{}, 0xc);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint32_t wave_sum(uint32_t v) { return wave_total(wave_scan_incl(v)); }

// Cross-wave combinations of per-wave values (nw <= 64 waves, `wave` the
// calling wave's index, uniform): lane w of every wave takes wave w's value,
// and one wave-wide DPP scan or reduction combines them -- no serial loop
// over the waves.  waves_before: sum of the values of waves < wave; total:
// sum of all.
__device__ __forceinline__ uint32_t waves_before(const uint32_t* per_wave, int nw, int wave, uint32_t& total) {
  const int lane = threadIdx.x & 63;
  const uint32_t x = per_wave[lane < nw ? lane : 0];
  const uint32_t incl = wave_scan_incl(lane < nw ? x : 0u);
  total = (uint32_t)__builtin_amdgcn_readlane((int)incl, nw - 1);
  const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)incl, wave > 0 ? wave - 1 : 0);
  return wave > 0 ? b : 0u;
}
__device__ __forceinline__ uint32_t waves_max(const uint32_t* per_wave, int nw) {
  const int lane = threadIdx.x & 63;
  const uint32_t x = per_wave[lane < nw ? lane : 0];
  return wave_max(lane < nw ? x : 0u);
}
__device__ __forceinline__ uint32_t waves_min(const uint32_t* per_wave, int nw) {
  const int lane = threadIdx.x & 63;
  const uint32_t x = per_wave[lane < nw ? lane : 0];
  return wave_min(lane < nw ? x : 0xFFFFFFFFu);
}

// The score threshold of an order-key threshold tau: for every score x
// (finite or -inf), order_key(x) >= tau exactly when x >= key_threshold(tau)
// (the key map is monotone in the score, -0 and +0 alike, and the inverse of
// a key is a float bit pattern); tau at or below the key of -inf admits every
// score.  NaN (a position past a row's end) passes no such test.
__device__ __forceinline__ float key_threshold(uint32_t tau) {
  return tau <= order_key(-__builtin_inff()) ? -__builtin_inff()
                                              : __uint_as_float((tau & 0x80000000u) ? (tau & 0x7FFFFFFFu) : ~tau);
}

// Sampling block of a row: B = kRun (every score) for short rows, else the
// smallest power of two >= 256 with vis / B * kRun <= kMaxSamples.
__device__ __forceinline__ int sample_block(int vis) {
  if (vis <= kExactMax) return kRun;
  int b = 256;
  while ((int64_t)b * kMaxSamples < (int64_t)vis * kRun) b <<= 1;
  return b;
}

// Block-wide inclusive suffix scan over nb = 4 * blockDim bins held 4 per
// thread (bins 4*tid .. 4*tid+3), then the bin holding rank r from the top:
// count(bins > b) < r <= count(bins >= b).  Every thread gets b and
// need = r - count(bins > b).  wtot: 16 words of LDS.
__device__ __forceinline__ void rank_bin_1024(const uint32_t* h, uint32_t r, uint32_t* wtot, int* s_bin,
                                              uint32_t* s_need, int& bin, uint32_t& need,
                                              uint32_t* s_count = nullptr, uint32_t* count = nullptr) {
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  uint32_t loc[4], sum = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    loc[i] = h[4 * tid + i];
    sum += loc[i];
  }
  // suffix sum over the lanes >= this one = wave total - prefix before it
  const uint32_t pre_incl = wave_scan_incl(sum);
  const uint32_t wt = wave_total(pre_incl);
  uint32_t suf = wt - pre_incl + sum;
  if (lane == 0) wtot[wave] = wt;
  __syncthreads();
  uint32_t all;
  const uint32_t before = waves_before(wtot, 16, wave, all);
  suf += all - before - wt;  // the waves after this one
  const uint32_t above = suf - sum;
  if (above < r && suf >= r) {
    uint32_t acc = above;
    for (int i = 3; i >= 0; --i) {
      if (acc + loc[i] >= r) {
        *s_bin = 4 * tid + i;
        *s_need = r - acc;
        if (s_count) *s_count = loc[i];
        break;
      }
      acc += loc[i];
    }
  }
  __syncthreads();
  bin = *s_bin;
  need = *s_need;
  if (s_count) *count = *s_count;
}

__global__ __launch_bounds__(1024) void topk_threshold_kernel(TopkParams p) {
  __shared__ uint32_t h[4096];
  __shared__ uint32_t wtot[16];
  __shared__ uint32_t s_lo[16], s_hi[16];
  __shared__ int s_bin;
  __shared__ uint32_t s_need;
  const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int vis = row_vis(p, t);
  uint32_t* ctr = p.ctr + (int64_t)t * 4;
  if (vis <= p.k) {
    if (tid < 4) ctr[tid] = 0;
    return;
  }
  const int B = sample_block(vis);
  const float* row = p.scores + (int64_t)t * p.ld;
  // sample keys (16 per thread, all loads issued first); 0 marks "no sample"
  // (below every finite or -inf score's key)
  uint32_t key[16];
  float v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int e = tid + 1024 * i;
    const int64_t s = (int64_t)(e / kRun) * B + (e % kRun);
    v[i] = s < vis ? row[s] : 0.f;
  }
  uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int e = tid + 1024 * i;
    const int64_t s = (int64_t)(e / kRun) * B + (e % kRun);
    key[i] = s < vis ? order_key(v[i]) : 0u;
    if (s < vis) {
      lo = min(lo, key[i]);
      hi = max(hi, key[i]);
    }
  }
  lo = wave_min(lo);
  hi = wave_max(hi);
  if (lane == 0) {
    s_lo[wave] = lo;
    s_hi[wave] = hi;
  }
  for (int i = tid; i < 4096; i += 1024) h[i] = 0;
  __syncthreads();
  lo = waves_min(s_lo, 16);
  hi = waves_max(s_hi, 16);
  // number of samples (blocks < kMaxSamples / kRun; the last may be partial)
  // and the rank of the threshold among them
  const int64_t nblk = ((int64_t)vis + B - 1) / B;
  const int64_t cb = min<int64_t>(nblk, kMaxSamples / kRun);
  const int64_t full = vis / B;  // blocks with all kRun samples present
  const int64_t S = min(full, cb) * kRun + (cb > full ? min<int64_t>(kRun, vis - full * B) : 0);
  uint32_t r;
  if (B == kRun) {
    r = (uint32_t)p.k;  // exact: the K-th largest key
  } else {
    const float mu = (float)p.k * (float)S / (float)vis;
    r = (uint32_t)min<int64_t>(S, (int64_t)ceilf(mu + 4.f * sqrtf(mu) + 8.f));
  }
  if (tid == 0) {  // a rank beyond the samples cannot happen; keep the result defined anyway
    s_bin = 0;
    s_need = 1;
  }
  // level 1: 12-bit bins over the sample's key range
  const uint32_t diff = lo ^ hi;
  const int nbits = diff ? 32 - __clz((int)diff) : 0;
  const int sh1 = max(nbits - 12, 0);
  const uint32_t base1 = lo >> sh1;
#pragma unroll
  for (int i = 0; i < 16; ++i)
    if (key[i] >= lo && key[i] != 0u) atomicAdd(&h[(key[i] >> sh1) - base1], 1u);
  __syncthreads();
  int b1;
  uint32_t need1;
  rank_bin_1024(h, r, wtot, &s_bin, &s_need, b1, need1);
  uint32_t tau = (base1 + (uint32_t)b1) << sh1;
  if (sh1 > 0) {
    // level 2: the next (up to) 12 bits inside bin b1
    const int sh2 = max(sh1 - 12, 0);
    const uint32_t mask2 = (1u << (sh1 - sh2)) - 1u;
    for (int i = tid; i < 4096; i += 1024) h[i] = 0;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (key[i] != 0u && (key[i] >> sh1) - base1 == (uint32_t)b1) atomicAdd(&h[(key[i] >> sh2) & mask2], 1u);
    __syncthreads();
    int b2;
    uint32_t need2;
    rank_bin_1024(h, need1, wtot, &s_bin, &s_need, b2, need2);
    tau |= (uint32_t)b2 << sh2;
  }
  if (tid == 0) {
    ctr[0] = 0;    // candidates appended by the filter
    ctr[1] = 0;
    ctr[2] = tau;  // keys >= tau are candidates
    ctr[3] = 0;
  }
}

// Keys >= tau of one slice, in index order: thread tid holds scores
// 4*tid + 1024*b + e (stripe b < 8, e < 4), so (b, tid, e) order is index
// order.  A block scan of the per-stripe counts (four 16-bit fields per
// 64-bit word, two words) gives every candidate its place; the slice's
// candidates go out as one contiguous block behind one global atomic, and
// the block's (base, count) is recorded for the finalize.
// (The words hold 16-bit fields whose sums never carry out of their field,
// so the two 32-bit halves are scanned independently.)
__device__ __forceinline__ uint64_t wave_scan_incl_u64(uint64_t v) {
  return (uint64_t)wave_scan_incl((uint32_t)v) | ((uint64_t)wave_scan_incl((uint32_t)(v >> 32)) << 32);
}
// 64-bit words whose 32-bit halves never carry into each other (16-bit
// fields): the halves are combined independently.
__device__ __forceinline__ uint64_t waves_before_u64(const uint64_t* per_wave, int nw, int wave, uint64_t& total) {
  const int lane = threadIdx.x & 63;
  const uint64_t y = per_wave[lane < nw ? lane : 0];
  const uint64_t x = lane < nw ? y : 0ull;
  const uint32_t il = wave_scan_incl((uint32_t)x), ih = wave_scan_incl((uint32_t)(x >> 32));
  total = (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)il, nw - 1) |
          ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)ih, nw - 1) << 32);
  const int src = wave > 0 ? wave - 1 : 0;
  const uint64_t b = (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)il, src) |
                     ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)ih, src) << 32);
  return wave > 0 ? b : 0ull;
}
__device__ __forceinline__ uint64_t block_excl_scan_u64(uint64_t v, uint64_t* wsum, uint64_t& total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint64_t inc = wave_scan_incl_u64(v);
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  const uint64_t before = waves_before_u64(wsum, (int)(blockDim.x >> 6), wave, total);
  return before + inc - v;
}

// NWD (<= 4) words at once, behind one barrier.  wsum: [16][4].
template <int NWD>
__device__ __forceinline__ void block_excl_scan_u64x4(const uint64_t (&v)[NWD], uint64_t (&ex)[NWD],
                                                      uint64_t (&tot)[NWD], uint64_t (*wsum)[4]) {
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  uint64_t inc[NWD];
#pragma unroll
  for (int i = 0; i < NWD; ++i) inc[i] = wave_scan_incl_u64(v[i]);
  if (lane == 63)
#pragma unroll
    for (int i = 0; i < NWD; ++i) wsum[wave][i] = inc[i];
  __syncthreads();
  const int nw = (int)(blockDim.x >> 6);
  const int ln = lane < nw ? lane : 0;
#pragma unroll
  for (int i = 0; i < NWD; ++i) {
    const uint64_t x = lane < nw ? wsum[ln][i] : 0ull;
    const uint32_t il = wave_scan_incl((uint32_t)x), ih = wave_scan_incl((uint32_t)(x >> 32));
    tot[i] = (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)il, nw - 1) |
             ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)ih, nw - 1) << 32);
    const int src = wave > 0 ? wave - 1 : 0;
    const uint64_t b = (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)il, src) |
                       ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)ih, src) << 32);
    ex[i] = inc[i] - v[i] + (wave > 0 ? b : 0ull);
  }
}

__global__ __launch_bounds__(256) void topk_filter_kernel(TopkParams p) {
  __shared__ uint64_t wsum[2][4];
  const int t = blockIdx.y;
  const int tid = threadIdx.x;
  const int vis = row_vis(p, t);
  if (vis <= p.k) return;
  const int s_begin = blockIdx.x * p.slice;
  const uint32_t* ctr = p.ctr + (int64_t)t * 4;
  uint32_t* info = p.slice_info + ((int64_t)t * p.nslices + blockIdx.x) * 2;
  if (s_begin >= vis) {
    if (tid == 0) {
      info[0] = 0;
      info[1] = 0;
    }
    return;
  }
  const int s_end = min(s_begin + p.slice, vis);
  const float* row = p.scores + (int64_t)t * p.ld;
  // The whole slice (8 float4 per thread) is loaded before any is compared:
  // every float4 read is issued unconditionally, a start past the row's ld
  // columns (ld and s_begin are multiples of 4) clamped to the last float4,
  // and positions at or past the slice end are masked afterwards (a read
  // under a branch made each wait for the one before).  The reads are
  // nontemporal (each score is read once; 256K FP4 batch: 51 -> 43 us).
  const int last4 = (int)min<int64_t>(p.ld - 4, INT32_MAX - 3);
  f32x4 v[8];
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const int s = s_begin + 4 * tid + 1024 * b;
    v[b] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(row + min(s, last4)));
  }
  const float tf = key_threshold(ctr[2]);
  uint32_t hit[8];  // bit e of hit[b]: score 4*tid + 1024*b + e is a candidate
  uint64_t pk[2] = {0, 0};
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    uint32_t m = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int s = s_begin + 4 * tid + 1024 * b + e;
      if (s < s_end && v[b][e] >= tf) m |= 1u << e;
    }
    hit[b] = m;
    pk[b >> 2] |= (uint64_t)__popc(m) << (16 * (b & 3));
  }
  uint64_t tot0, tot1;
  const uint64_t ex0 = block_excl_scan_u64(pk[0], wsum[0], tot0);
  const uint64_t ex1 = block_excl_scan_u64(pk[1], wsum[1], tot1);
  // stripe totals -> stripe offsets
  uint32_t off[8], n = 0;
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    off[b] = n;
    n += (uint32_t)(((b < 4 ? tot0 : tot1) >> (16 * (b & 3))) & 0xFFFFu);
  }
  // the slice's own region (slice_cap entries; a count above it sends the
  // row to the whole-row selection)
  if (tid == 0) {
    info[0] = 0;
    info[1] = n;
  }
  uint32_t* creg = p.cand + ((int64_t)t * p.nslices + blockIdx.x) * p.slice_cap * 2;
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    uint32_t pos = off[b] + (uint32_t)(((b < 4 ? ex0 : ex1) >> (16 * (b & 3))) & 0xFFFFu);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (hit[b] >> e & 1u) {
        if (pos < (uint32_t)p.slice_cap) {
          const int s = s_begin + 4 * tid + 1024 * b + e;
          creg[2 * pos] = order_key(v[b][e]);
          creg[2 * pos + 1] = (uint32_t)s;
        }
        ++pos;
      }
    }
  }
}

__device__ __forceinline__ uint64_t composite(uint32_t key, uint32_t idx) {
  return ((uint64_t)key << 32) | (uint64_t)(0xFFFFFFFFu - idx);
}

// Logical index li of request r -> physical row page * P + slot, or -1 for
// no index or no request, an index past the request's block-table row, or a
// page outside [0, num_pages) (an absent page: nothing of it may be read).
__device__ __forceinline__ int translate_one(int li, int r, const int32_t* __restrict__ bt, int bt_stride,
                                             int plog2, int num_pages) {
  if (li < 0 || r < 0) return -1;
  const int lp = li >> plog2;
  int pg;
  if (bt) {
    DSA_DEBUG_NOTE(lp >= bt_stride, DSA_DEBUG_ROW_OUTSIDE);
    if (lp >= bt_stride) return -1;
    pg = bt[(int64_t)r * bt_stride + lp];
  } else {
    pg = r;
  }
  DSA_DEBUG_NOTE(pg < 0 || pg >= num_pages, DSA_DEBUG_ABSENT_PAGE);
  if (pg < 0 || pg >= num_pages) return -1;
  return (pg << plog2) | (li & ((1 << plog2) - 1));
}

// Shared scratch of the 1024-thread selection and sort.
struct SelectLds {
  uint32_t h[4096];
  uint32_t wtot[16];
  uint64_t red[2][16];
  int bin, cnt;
  uint32_t need, hcount;
};

// Exact selection of the K largest among distinct 64-bit composites that the
// workgroup's 1024 threads enumerate (each(f) calls f(v) for every composite
// of the calling thread): radix select with 12-bit digits, starting at the
// highest bit in which the composites differ.  On return, v is a winner iff
// (v >> hi_sh) >= prefix; exactly K composites are.
template <class Each>
__device__ __forceinline__ void select_top(Each each, uint32_t K, SelectLds& sl, int& hi_sh_out,
                                           uint64_t& prefix_out) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint64_t mx = 0, mn = ~0ull;
  each([&](uint64_t v) {
    mx = v > mx ? v : mx;
    mn = v < mn ? v : mn;
  });
  mx = wave_max_u64(mx);
  mn = ~wave_max_u64(~mn);
  if (lane == 0) {
    sl.red[0][wave] = mx;
    sl.red[1][wave] = mn;
  }
  __syncthreads();
  {
    const int ln = lane < 16 ? lane : 0;
    const uint64_t a = sl.red[0][ln], b = sl.red[1][ln];
    mx = wave_max_u64(lane < 16 ? a : 0ull);
    mn = ~wave_max_u64(lane < 16 ? ~b : 0ull);
  }
  const uint64_t dif = mx ^ mn;
  int hi_sh = dif ? 64 - __clzll((long long)dif) : 1;  // bits >= hi_sh: common prefix
  uint64_t prefix = hi_sh >= 64 ? 0ull : (mx >> hi_sh);
  uint32_t need = K;
  for (;;) {
    const int lo_sh = max(hi_sh - 12, 0);
    const uint64_t dmask = (1ull << (hi_sh - lo_sh)) - 1ull;
    for (int i = tid; i < 4096; i += 1024) sl.h[i] = 0;
    if (tid == 0) {
      sl.bin = 0;
      sl.need = 1;
      sl.hcount = 1;
    }
    __syncthreads();
    each([&](uint64_t v) {
      const uint64_t pre = hi_sh >= 64 ? 0ull : (v >> hi_sh);
      if (pre == prefix) atomicAdd(&sl.h[(v >> lo_sh) & dmask], 1u);
    });
    __syncthreads();
    int b;
    uint32_t nn, hv;
    rank_bin_1024(sl.h, need, sl.wtot, &sl.bin, &sl.need, b, nn, &sl.hcount, &hv);
    prefix = (prefix << (hi_sh - lo_sh)) | (uint64_t)b;
    hi_sh = lo_sh;
    need = nn;
    if (hv == nn || lo_sh == 0) break;
  }
  hi_sh_out = hi_sh;
  prefix_out = prefix;
}

// Order the K winners in out[0..K) by index and write idx / physical rows of
// row t.  An LDS bitmap (bm, bm_words words) covers a window of the index
// range, W words per thread; a block prefix sum of the threads' popcounts
// gives every winner its rank directly (rank = set bits before it), so no
// thread walks its bits one by one.  Windows repeat until vis is covered.
// ord: LDS int[2048] (the ordered list), tpre: LDS int[1024], wsum: 16 words.
__device__ __forceinline__ void order_and_store(const TopkParams& p, const int* out, int K, int vis, uint32_t* bm,
                                                int bm_words, int* ord, int* tpre, uint32_t* wsum, int t, int r,
                                                int32_t* idx, int32_t* rows) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int need_words = (vis + 31) >> 5;
  const int W = max(1, min(bm_words >> 10, (need_words + 1023) >> 10));
  const int win = W * 1024 * 32;
  int emitted = 0;
  for (int w0 = 0; w0 < vis; w0 += win) {
    for (int i = 0; i < W; ++i) bm[tid * W + i] = 0;
    __syncthreads();
    for (int j = tid; j < K; j += 1024) {
      const int li = out[j] - w0;
      if (li >= 0 && li < win) atomicOr(&bm[li >> 5], 1u << (li & 31));
    }
    __syncthreads();
    int cnt = 0;
    for (int i = 0; i < W; ++i) cnt += __popc(bm[tid * W + i]);
    const int inc = (int)wave_scan_incl((uint32_t)cnt);
    if (lane == 63) wsum[wave] = (uint32_t)inc;
    __syncthreads();
    int before = inc - cnt, tot = 0;
    for (int w = 0; w < 16; ++w) {
      if (w < wave) before += (int)wsum[w];
      tot += (int)wsum[w];
    }
    tpre[tid] = before;
    __syncthreads();
    for (int j = tid; j < K; j += 1024) {
      const int li = out[j] - w0;
      if (li >= 0 && li < win) {
        const int w = li >> 5, own = w / W;
        int rk = tpre[own] + __popc(bm[w] & ((1u << (li & 31)) - 1u));
        for (int x = own * W; x < w; ++x) rk += __popc(bm[x]);
        ord[emitted + rk] = out[j];
      }
    }
    emitted += tot;
    __syncthreads();
  }
  // coalesced stores; the block-table reads of all entries are in flight at once
  for (int j = tid; j < p.k; j += 1024) {
    const int li = j < K ? ord[j] : -1;
    idx[j] = li;
    if (rows) rows[j] = translate_one(li, r, p.block_table, p.bt_stride, p.plog2, p.num_pages);
  }
  if (p.count && tid == 0) p.count[t] = K;
}

// A row with vis <= k keeps every position.
__device__ __forceinline__ void store_all(const TopkParams& p, int vis, int t, int r, int32_t* idx, int32_t* rows) {
  if (vis <= 0 && p.skip_empty) return;
  for (int j = threadIdx.x; j < p.k; j += blockDim.x) {
    const int li = j < vis ? j : -1;
    idx[j] = li;
    if (rows) rows[j] = translate_one(li, r, p.block_table, p.bt_stride, p.plog2, p.num_pages);
  }
  if (p.count && threadIdx.x == 0) p.count[t] = vis;
}

// Dynamic LDS of the finalize: candidate keys [kTopkFinalCap] and indices
// [kTopkFinalCap] (later the ordering bitmap), the winners [2048], the
// ordered winners [2048], per-thread prefix sums [1024].
constexpr size_t kFinalLds = (size_t)2 * kTopkFinalCap * 4 + 2 * DSA_MAX_TOPK * 4 + 1024 * 4;

__global__ __launch_bounds__(1024) void topk_finalize_kernel(TopkParams p) {
  extern __shared__ uint32_t fsm[];
  uint32_t* ck = fsm;
  uint32_t* ci = fsm + kTopkFinalCap;
  int* out = reinterpret_cast<int*>(fsm + 2 * kTopkFinalCap);
  int* ord = out + DSA_MAX_TOPK;
  int* tpre = ord + DSA_MAX_TOPK;
  __shared__ SelectLds sl;
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int vis = row_vis(p, t);
  const int K = min(p.k, vis);
  const int r = row_req(p, t);
  int32_t* idx = p.idx + (int64_t)t * p.k;
  int32_t* rows = p.rows ? p.rows + (int64_t)t * p.k : nullptr;
  if (vis <= p.k) {
    store_all(p, vis, t, r, idx, rows);
    return;
  }

  // Slice counts (rows of up to 1024 slices, 8M scores), their exclusive
  // prefix, and the candidates gathered from the slices' regions into LDS in
  // index order; the whole score row instead when the estimate missed (fewer
  // than K, or more than the LDS or a slice's region holds).
  const float* srow = p.scores + (int64_t)t * p.ld;
  uint32_t* soff = reinterpret_cast<uint32_t*>(ord);  // [nslices <= 1024]
  uint32_t* scnt = reinterpret_cast<uint32_t*>(tpre);  // [nslices <= 1024]
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool sliced = p.nslices <= 1024;
  int ncand = 0;
  bool over = !sliced;
  if (sliced) {
    const uint32_t* info = p.slice_info + (int64_t)t * p.nslices * 2;
    const uint32_t cnt = tid < p.nslices ? info[2 * tid + 1] : 0u;
    const int inc = (int)wave_scan_incl(cnt);
    const bool big = __ballot(cnt > (uint32_t)p.slice_cap) != 0;
    if (lane == 63) sl.wtot[wave] = (uint32_t)inc;
    if (lane == 0) sl.h[wave] = big ? 1u : 0u;
    __syncthreads();
    uint32_t all;
    const int before = (int)waves_before(sl.wtot, 16, wave, all);
    ncand = (int)all;
    over = waves_max(sl.h, 16) != 0u;
    if (tid < p.nslices) {
      soff[tid] = (uint32_t)(before + inc) - cnt;
      scnt[tid] = cnt;
    }
  }
  const bool from_row = over || ncand < K || ncand > p.cand_cap;
  const int nsrc = from_row ? vis : ncand;
  const bool ordered = !from_row;
  __syncthreads();
  if (ordered) {
    // wave w copies slices w, w + 16, ...; its lanes take consecutive entries
    for (int sidx = wave; sidx < p.nslices; sidx += 16) {
      const int n = (int)scnt[sidx], o = (int)soff[sidx];
      const uint2* creg = reinterpret_cast<const uint2*>(p.cand + ((int64_t)t * p.nslices + sidx) * p.slice_cap * 2);
      for (int j = lane; j < n; j += 64) {
        const uint2 cv = creg[j];
        ck[o + j] = cv.x;
        ci[o + j] = cv.y;
      }
    }
  }
  __syncthreads();
  auto each = [&](auto f) {
    for (int i = tid; i < nsrc; i += 1024)
      f(from_row ? composite(order_key(srow[i]), (uint32_t)i) : composite(ck[i], ci[i]));
  };
  int hi_sh;
  uint64_t prefix;
  select_top(each, (uint32_t)K, sl, hi_sh, prefix);
  if (ordered) {
    // the candidates are in index order: a stable compaction of the winners
    // (thread tid owns candidates 8*tid .. 8*tid+7) is the ordered result
    constexpr int kPer = kTopkFinalCap / 1024;
    uint32_t m = 0;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int i = kPer * tid + u;
      if (i < ncand && (composite(ck[i], ci[i]) >> hi_sh) >= prefix) m |= 1u << u;
    }
    const int inc = (int)wave_scan_incl((uint32_t)__popc(m));
    __syncthreads();  // sl.wtot was read by select_top
    if (lane == 63) sl.wtot[wave] = (uint32_t)inc;
    __syncthreads();
    uint32_t all_unused;
    int pos = inc - __popc(m) + (int)waves_before(sl.wtot, 16, wave, all_unused);
#pragma unroll
    for (int u = 0; u < kPer; ++u)
      if (m >> u & 1u) ord[pos++] = (int)ci[kPer * tid + u];
    __syncthreads();
    for (int j = tid; j < p.k; j += 1024) {
      const int li = j < K ? ord[j] : -1;
      idx[j] = li;
      if (rows) rows[j] = translate_one(li, r, p.block_table, p.bt_stride, p.plog2, p.num_pages);
    }
    if (p.count && tid == 0) p.count[t] = K;
    return;
  }
  if (tid == 0) sl.cnt = 0;
  __syncthreads();
  each([&](uint64_t v) {
    if ((v >> hi_sh) >= prefix) {
      const int pos = atomicAdd(&sl.cnt, 1);
      if (pos < DSA_MAX_TOPK) out[pos] = (int)(0xFFFFFFFFu - (uint32_t)v);
    }
  });
  __syncthreads();
  order_and_store(p, out, K, vis, fsm, 2 * kTopkFinalCap, ord, tpre, sl.wtot, t, r, idx, rows);
}

// Rows up to kRowMax scores: one workgroup per row does everything with the
// row held in registers (NS float4 per thread: scores 4*tid + 4096*i + c, so
// index order is (i, tid, c); NS = 16, or 8 for rows up to 32K, which halves
// the registers and the per-score work of the prefill shape, or 4 for rows
// up to 8K), one read of the row, one launch, no workspace.
//   threshold  from the sample key[tid & (NS-1)][*] (every NS-th group of four
//              scores; every score of a row up to the candidate capacity) by two 12-bit
//              histogram levels, as in the threshold kernel;
//   select     the exact radix select runs directly over the register keys
//              at or above the threshold (over all keys of the row when fewer
//              than K are: the estimate only decides speed);
//   order      winners are re-identified in registers and written in index
//              order: their per-stripe counts, packed four 16-bit fields to a
//              64-bit word, get one block exclusive scan.
constexpr int kRowMax = 16 * 4096;

// Candidates the per-row kernel holds in LDS: 8192 for rows up to 64K, 4096
// for rows up to 32K (about 2600 expected), whose workgroup then fits two to a
// CU (75 KB of LDS, 59 registers), and 8192 for rows up to 8K (four stripes):
// such a row is kept whole, with no sampled threshold, and every thread
// compares 16 register scores instead of 32.
template <int NS> constexpr int row_cap() { return NS == 8 ? 4096 : 8192; }

template <int CAP>
struct RowLdsT {
  SelectLds sl;
  uint32_t h2[4096];          // level-2 histogram (cleared with level 1's)
  uint32_t ck[CAP];           // candidate scores (bits), in index order
  uint32_t ci[CAP];           // their indices
  int ord[DSA_MAX_TOPK];      // the winners in index order
  uint32_t s_lo[16], s_hi[16];
  int s_cnt[16];
  uint64_t wsum4[16][4];
};

// Block exclusive scan of one int per thread (1024 threads); wsum: 16 ints.
__device__ __forceinline__ int block_excl_scan_i32(int v, int* wsum, int& total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int inc = (int)wave_scan_incl((uint32_t)v);
  __syncthreads();  // wsum may still be read by a previous scan
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  uint32_t tot;
  const int before = (int)waves_before(reinterpret_cast<const uint32_t*>(wsum), 16, wave, tot);
  total = (int)tot;
  return before + inc - v;
}

// Exact K-th largest among n keys get(0 .. n-1) (32-bit radix select, 12-bit
// digits from the highest bit in which they differ).  Afterwards the keys
// with (key >> sh) > pre win, and: full -> every key with (key >> sh) == pre
// wins too; else (sh == 0) the first `need` keys equal to pre win.
template <class Get, class RowLds>
__device__ __forceinline__ void select32(Get get, int n, uint32_t K, RowLds& L, int& sh_out, uint32_t& pre_out,
                                         uint32_t& need_out, bool& full_out) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t mx = 0, mn = 0xFFFFFFFFu;
  for (int j = tid; j < n; j += 1024) {
    const uint32_t k2 = get(j);
    mx = max(mx, k2);
    mn = min(mn, k2);
  }
  mx = wave_max(mx);
  mn = wave_min(mn);
  __syncthreads();
  if (lane == 0) {
    L.s_lo[wave] = mn;
    L.s_hi[wave] = mx;
  }
  __syncthreads();
  mn = waves_min(L.s_lo, 16);
  mx = waves_max(L.s_hi, 16);
  const uint32_t dif = mx ^ mn;
  int sh = dif ? 32 - __clz((int)dif) : 0;
  uint32_t pre = sh >= 32 ? 0u : (mx >> sh);
  uint32_t need = K;
  bool full = true;
  while (sh > 0) {
    const int lo_sh = max(sh - 12, 0);
    const uint32_t dmask = (1u << (sh - lo_sh)) - 1u;
    for (int i = tid; i < 4096; i += 1024) L.sl.h[i] = 0;
    if (tid == 0) {
      L.sl.bin = 0;
      L.sl.need = 1;
      L.sl.hcount = 1;
    }
    __syncthreads();
    for (int j = tid; j < n; j += 1024) {
      const uint32_t k2 = get(j);
      if ((sh >= 32 ? 0u : (k2 >> sh)) == pre) atomicAdd(&L.sl.h[(k2 >> lo_sh) & dmask], 1u);
    }
    __syncthreads();
    int bsel;
    uint32_t nn, hv;
    rank_bin_1024(L.sl.h, need, L.sl.wtot, &L.sl.bin, &L.sl.need, bsel, nn, &L.sl.hcount, &hv);
    pre = (sh >= 32 ? 0u : (pre << (sh - lo_sh))) | (uint32_t)bsel;
    sh = lo_sh;
    need = nn;
    full = hv == nn;
    if (full) break;
  }
  sh_out = sh;
  pre_out = pre;
  need_out = need;
  full_out = full;
}

// The winners of select32 among get(0 .. n-1), in index order, into ord[]:
// chunks of 8192 keys, thread tid owning keys 8 tid .. 8 tid + 7 of a chunk;
// block scans of the counts of equal keys (the tie-break rank) and of
// winners, carried from chunk to chunk.
template <class Get, class Idx, class RowLds>
__device__ __forceinline__ void emit_winners(Get get, Idx index_of, int n, int sh, uint32_t pre, uint32_t need,
                                             bool full, RowLds& L) {
  const int tid = threadIdx.x;
  int eq_carry = 0, win_carry = 0;
  for (int base = 0; base < n; base += 8 * 1024) {
    const int j0 = base + 8 * tid;
    uint32_t kv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) kv[u] = j0 + u < n ? get(j0 + u) : 0u;
    uint32_t wmask = 0;
    if (full) {
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (j0 + u < n && (kv[u] >> sh) >= pre) wmask |= 1u << u;
    } else {
      int e = 0;
#pragma unroll
      for (int u = 0; u < 8; ++u) e += (j0 + u < n && kv[u] == pre) ? 1 : 0;
      int etot;
      int rk = eq_carry + block_excl_scan_i32(e, L.s_cnt, etot);
      eq_carry += etot;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (j0 + u >= n) continue;
        if (kv[u] > pre) {
          wmask |= 1u << u;
        } else if (kv[u] == pre) {
          if ((uint32_t)rk < need) wmask |= 1u << u;
          ++rk;
        }
      }
    }
    int wtot;
    int pos = win_carry + block_excl_scan_i32(__popc(wmask), L.s_cnt, wtot);
    win_carry += wtot;
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (wmask >> u & 1u) L.ord[pos++] = index_of(j0 + u);
  }
  __syncthreads();
}

template <int NS>
__global__ __launch_bounds__(1024) void topk_row_kernel(TopkParams p) {
  constexpr int kRowCap = row_cap<NS>();
  __shared__ RowLdsT<kRowCap> L;
  const int t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int vis = row_vis(p, t);
  const int K = min(p.k, vis);
  const int r = row_req(p, t);
  int32_t* idx = p.idx + (int64_t)t * p.k;
  int32_t* rows = p.rows ? p.rows + (int64_t)t * p.k : nullptr;
  if (vis <= p.k) {
    store_all(p, vis, t, r, idx, rows);
    return;
  }
  // Every float4 read is issued, unconditionally: a start past the row's ld
  // columns (ld is a multiple of 4) is clamped to the last float4 and its
  // values are masked, so no read waits behind a branch.  The reads are
  // nontemporal (each score is read once; cached reads also paid for
  // evicting other dirty lines: the row's read 17.6 -> 11.2 us at 64K).
  // The scores stay floats: a position at or past vis holds NaN, which no
  // comparison admits (scores are finite or -inf), and the order key of a
  // score is formed only for the sample and the candidates.
  f32x4 x[NS];
  {
    const float* row = p.scores + (int64_t)t * p.ld;
    const int last4 = (int)min<int64_t>(p.ld - 4, NS * 4096 - 4);
#pragma unroll
    for (int i = 0; i < NS; ++i)
      x[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(row + min(4 * tid + 4096 * i, last4)));
#pragma unroll
    for (int i = 0; i < NS; ++i)
      if (4096 * (i + 1) > vis)  // (uniform) stripe i reaches past vis
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (4 * tid + 4096 * i + c >= vis) x[i][c] = __builtin_nanf("");
  }
  auto key_of = [](float v) { return v == v ? order_key(v) : 0u; };  // 0: past vis
  for (int i = tid; i < 4096; i += 1024) {
    L.sl.h[i] = 0;
    L.h2[i] = 0;
  }
  if (tid == 0) {
    L.sl.bin = 0;
    L.sl.need = 1;
  }

  // ---- threshold: keys >= tau are the candidates (tau = 1: every key)
  uint32_t tau = 1u;
  if (vis > kRowCap) {  // (a row up to the candidate capacity keeps every score)
    uint32_t samp[4];
    const int sel = tid & (NS - 1);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      float v = x[0][c];
#pragma unroll
      for (int i = 1; i < NS; ++i) v = sel == i ? x[i][c] : v;
      samp[c] = key_of(v);
    }
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
    int ns = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (samp[c] != 0u) {
        lo = min(lo, samp[c]);
        hi = max(hi, samp[c]);
        ++ns;
      }
    lo = wave_min(lo);
    hi = wave_max(hi);
    ns = (int)wave_sum((uint32_t)ns);
    if (lane == 0) {
      L.s_lo[wave] = lo;
      L.s_hi[wave] = hi;
      L.s_cnt[wave] = ns;
    }
    __syncthreads();
    lo = waves_min(L.s_lo, 16);
    hi = waves_max(L.s_hi, 16);
    uint32_t S_all;
    (void)waves_before(reinterpret_cast<const uint32_t*>(L.s_cnt), 16, 0, S_all);
    const int S = (int)S_all;
    const float mu = (float)K * (float)S / (float)vis;
    const uint32_t rk = (uint32_t)min<int64_t>(S, (int64_t)ceilf(mu + 4.f * sqrtf(mu) + 8.f));
    const uint32_t diff = lo ^ hi;
    const int nbits = diff ? 32 - __clz((int)diff) : 0;
    const int sh1 = max(nbits - 12, 0);
    const uint32_t base1 = lo >> sh1;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (samp[c] != 0u) atomicAdd(&L.sl.h[(samp[c] >> sh1) - base1], 1u);
    __syncthreads();
    int b1;
    uint32_t need1;
    rank_bin_1024(L.sl.h, rk, L.sl.wtot, &L.sl.bin, &L.sl.need, b1, need1);
    tau = (base1 + (uint32_t)b1) << sh1;
    if (sh1 > 0) {
      const int sh2 = max(sh1 - 12, 0);
      const uint32_t mask2 = (1u << (sh1 - sh2)) - 1u;
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (samp[c] != 0u && (samp[c] >> sh1) - base1 == (uint32_t)b1) atomicAdd(&L.h2[(samp[c] >> sh2) & mask2], 1u);
      __syncthreads();
      int b2;
      uint32_t need2;
      rank_bin_1024(L.h2, need1, L.sl.wtot, &L.sl.bin, &L.sl.need, b2, need2);
      tau |= (uint32_t)b2 << sh2;
    }
    tau = max(tau, 1u);
  }

  // ---- candidates (keys >= tau) into LDS in index order: stripe i's count
  // in 16-bit field i & 3 of word i >> 2 (a stripe holds at most 4096 keys,
  // so fields never carry), one block exclusive scan per word.  key >= tau is
  // tested on the score itself.
  const float tf = key_threshold(tau);
  auto field = [](const uint64_t (&w)[NS / 4], int i) { return (uint32_t)((w[i >> 2] >> (16 * (i & 3))) & 0xFFFFu); };
  {
    constexpr int NWD = NS / 4;  // 64-bit words of four 16-bit stripe fields
    uint64_t pc[NWD], exc[NWD], totc[NWD];
#pragma unroll
    for (int w = 0; w < NWD; ++w) pc[w] = 0;
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      int n = 0;
#pragma unroll
      for (int c = 0; c < 4; ++c) n += x[i][c] >= tf ? 1 : 0;
      pc[i >> 2] |= (uint64_t)n << (16 * (i & 3));
    }
    block_excl_scan_u64x4(pc, exc, totc, L.wsum4);
    uint32_t ncand = 0;
#pragma unroll
    for (int i = 0; i < NS; ++i) ncand += field(totc, i);
    if (ncand >= (uint32_t)K && ncand <= (uint32_t)kRowCap) {
      uint32_t off = 0;
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        uint32_t pos = off + field(exc, i);
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (x[i][c] >= tf) {
            L.ck[pos] = __float_as_uint(x[i][c]);  // the score's bits (its order key is formed when read)
            L.ci[pos] = (uint32_t)(4 * tid + 4096 * i + c);
            ++pos;
          }
        off += field(totc, i);
      }
      __syncthreads();
      // ---- exact select over the candidates, and the winners in order
      int sh;
      uint32_t pre, need;
      bool full;
      const uint32_t* ck = L.ck;
      const uint32_t* ci = L.ci;
      auto ckey = [&](int j) { return order_key(__uint_as_float(ck[j])); };
      select32(ckey, (int)ncand, (uint32_t)K, L, sh, pre, need, full);
      emit_winners(ckey, [&](int j) { return (int)ci[j]; }, (int)ncand, sh, pre, need, full, L);
      for (int j = tid; j < p.k; j += 1024) {
        const int li = j < K ? L.ord[j] : -1;
        idx[j] = li;
        if (rows) rows[j] = translate_one(li, r, p.block_table, p.bt_stride, p.plog2, p.num_pages);
      }
      if (p.count && tid == 0) p.count[t] = K;
      return;
    }
  }
  // ---- the estimate missed (fewer than K or more than kRowCap candidates):
  // select over the whole row, read again from memory (rare)
  {
    const float* row = p.scores + (int64_t)t * p.ld;
    auto get = [&](int j) { return order_key(row[j]); };
    int sh;
    uint32_t pre, need;
    bool full;
    select32(get, vis, (uint32_t)K, L, sh, pre, need, full);
    emit_winners(get, [](int j) { return j; }, vis, sh, pre, need, full, L);
  }
  for (int j = tid; j < p.k; j += 1024) {
    const int li = j < K ? L.ord[j] : -1;
    idx[j] = li;
    if (rows) rows[j] = translate_one(li, r, p.block_table, p.bt_stride, p.plog2, p.num_pages);
  }
  if (p.count && tid == 0) p.count[t] = K;
}

// Rows up to kShortMax scores: one 256-thread workgroup per row holds the row
// in registers (32 consecutive scores per thread), finds the K-th largest key
// by an 8-bit radix select (early exit once the chosen bin is taken whole),
// and emits the winners in index order: all keys above the threshold digit
// prefix plus the first rho keys equal to it (lower indices first), placed by
// one block scan of the per-thread counts.  Little LDS, so many rows share a
// CU: this is the path for short rows (one 8K row, or many context-shard rows).
constexpr int kShortMax = 8192;
constexpr int kShortThreads = 256;
constexpr int kShortPer = kShortMax / kShortThreads;  // 32, one run per thread
constexpr int kShortMinRows = 512;                     // rows to fill the device twice over

__global__ __launch_bounds__(kShortThreads) void topk_short_kernel(TopkParams p) {
  __shared__ RadixLds<uint32_t, kShortThreads> L;
  const int t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int vis = row_vis(p, t);
  const int K = min(p.k, vis);
  const int r = row_req(p, t);
  int32_t* idx = p.idx + (int64_t)t * p.k;
  int32_t* rows = p.rows ? p.rows + (int64_t)t * p.k : nullptr;
  if (vis <= p.k) {
    store_all(p, vis, t, r, idx, rows);
    return;
  }
  // Loads: float4 q covers scores j0+4q .. j0+4q+3; it is issued only when its
  // first score is visible, and then lies inside the row (ld and j0+4q are
  // multiples of 4, j0+4q < vis <= ld).  Key 0 marks "no score" (no finite
  // score has key 0).
  const float* row = p.scores + (int64_t)t * p.ld;
  const int j0 = tid * kShortPer;
  uint32_t key[kShortPer];
#pragma unroll
  for (int q = 0; q < kShortPer / 4; ++q) {
    float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
    if (j0 + 4 * q < vis) x = *reinterpret_cast<const float4*>(row + j0 + 4 * q);
    key[4 * q + 0] = j0 + 4 * q + 0 < vis ? order_key(x.x) : 0u;
    key[4 * q + 1] = j0 + 4 * q + 1 < vis ? order_key(x.y) : 0u;
    key[4 * q + 2] = j0 + 4 * q + 2 < vis ? order_key(x.z) : 0u;
    key[4 * q + 3] = j0 + 4 * q + 3 < vis ? order_key(x.w) : 0u;
  }
  auto each = [&](auto f) {
#pragma unroll
    for (int i = 0; i < kShortPer; ++i) f(key[i]);
  };
  uint32_t prefix;
  int shift, rho;
  radix_kth<uint32_t, kShortThreads>(each, K, L, prefix, shift, rho);
  const uint32_t P = shr_sat<uint32_t>(prefix, shift);
  uint32_t gt = 0, eq = 0;
  each([&](uint32_t k) {
    if (k != 0) {
      gt += shr_sat<uint32_t>(k, shift) > P;
      eq += shr_sat<uint32_t>(k, shift) == P;
    }
  });
  // exclusive scan of (gt, eq) packed in 16-bit halves (each total <= 8192)
  const uint32_t v = (gt << 16) | eq;
  uint32_t inc = wave_scan_incl(v);
  if (lane == 63) L.wsum[wave] = inc;  // (the selection read wsum before its final barrier)
  __syncthreads();
  for (int w = 0; w < wave; ++w) inc += L.wsum[w];
  const uint32_t ex = inc - v;
  const int eq_before = (int)(ex & 0xFFFFu);
  int pos = (int)(ex >> 16) + min(eq_before, rho);
  int eqi = eq_before;
#pragma unroll
  for (int i = 0; i < kShortPer; ++i) {
    if (key[i] != 0) {
      const uint32_t kk = shr_sat<uint32_t>(key[i], shift);
      const bool take = kk > P || (kk == P && eqi < rho);
      eqi += kk == P;
      if (take) {
        const int j = j0 + i;
        idx[pos] = j;
        if (rows) rows[pos] = translate_one(j, r, p.block_table, p.bt_stride, p.plog2, p.num_pages);
        ++pos;
      }
    }
  }
  for (int j = K + tid; j < p.k; j += kShortThreads) {
    idx[j] = -1;
    if (rows) rows[j] = -1;
  }
  if (p.count && tid == 0) p.count[t] = K;
}

__global__ void translate_kernel(const int32_t* __restrict__ idx, int k, int T, const int32_t* __restrict__ tok_req,
                                 int R, const int32_t* __restrict__ bt, int bt_stride, int plog2, int num_pages,
                                 int32_t* __restrict__ rows) {
  const int64_t n = (int64_t)T * k;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int t = (int)(i / k);
    rows[i] = translate_one(idx[i], req_or_none(tok_req[t], R), bt, bt_stride, plog2, num_pages);
  }
}

dsa_status launch_topk(const TopkParams& p, hipStream_t stream) {
  // (few short rows: the 1024-thread row kernel has the shorter per-row latency)
  if (p.max_vis <= kShortMax && p.T >= kShortMinRows) {
    hipLaunchKernelGGL(topk_short_kernel, dim3(p.T), dim3(kShortThreads), 0, stream, p);
    return hipGetLastError() == hipSuccess ? DSA_OK : DSA_ERR_HIP;
  }
  if (p.max_vis <= row_cap<4>()) {
    hipLaunchKernelGGL((topk_row_kernel<4>), dim3(p.T), dim3(1024), 0, stream, p);
    return hipGetLastError() == hipSuccess ? DSA_OK : DSA_ERR_HIP;
  }
  if (p.max_vis <= kRowMax / 2) {
    hipLaunchKernelGGL((topk_row_kernel<8>), dim3(p.T), dim3(1024), 0, stream, p);
    return hipGetLastError() == hipSuccess ? DSA_OK : DSA_ERR_HIP;
  }
  if (p.max_vis <= kRowMax) {
    hipLaunchKernelGGL((topk_row_kernel<16>), dim3(p.T), dim3(1024), 0, stream, p);
    return hipGetLastError() == hipSuccess ? DSA_OK : DSA_ERR_HIP;
  }
  hipLaunchKernelGGL(topk_threshold_kernel, dim3(p.T), dim3(1024), 0, stream, p);
  hipLaunchKernelGGL(topk_filter_kernel, dim3(p.nslices, p.T), dim3(256), 0, stream, p);
  hipLaunchKernelGGL(topk_finalize_kernel, dim3(p.T), dim3(1024), kFinalLds, stream, p);
  return hipGetLastError() == hipSuccess ? DSA_OK : DSA_ERR_HIP;
}

dsa_status launch_translate(const int32_t* idx, int k, int T, const int32_t* tok_req, int R,
                            const int32_t* block_table, int bt_stride, int plog2, int num_pages, int32_t* rows, hipStream_t stream) {
  const int64_t n = (int64_t)T * k;
  hipLaunchKernelGGL(translate_kernel, dim3((unsigned)std::min<int64_t>((n + 255) / 256, 8192)), dim3(256), 0,
                     stream, idx, k, T, tok_req, R, block_table, bt_stride, plog2, num_pages, rows);
  return hipGetLastError() == hipSuccess ? DSA_OK : DSA_ERR_HIP;
}

DSA_DEBUG_TAKE(topk)

}  // namespace dsa
