// Per-row top-k with a lower-index tie-break, and block-table translation.
//
// Kimi K3.1 Pro day-0 page: "Sparse attention in K3.1 Pro" keeps the 2,048
// best-scored tokens per query; "Exact top-k merge" selects by radix select;
// AMD "Communication" asks for a consistent tie-break rule.  The set kept for
// row t is unique: the K = min(k, vis) largest scores, equal scores ordered by
// ascending index.  It is emitted in ascending index order.
//
// Two passes over the scores of a row, each spread over many workgroups:
//   1. histogram of the top 12 bits of the order-preserving uint32 key;
//   2. every slice finds the threshold bin b holding rank K from the row's
//      histogram and gathers keys above b ("definite", fewer than K in total)
//      and keys inside b ("candidates") in LDS and appends them to per-row
//      buffers behind one global atomic per list;
//   3. one workgroup per row refines the candidates (in LDS) with an exact
//      radix select on the 56-bit composite (low 20 key bits, then inverted
//      index), so ties resolve to the lower index, then orders the K winners
//      by index through an LDS bitmap (popcount prefix sums) and writes
//      indices, physical rows and the count.
// If a row's candidates overflow their buffer, step 3 reads them straight
// from the score row instead (slower, same result).
#include "common.h"
#include "kernels.h"

namespace dsa {

constexpr int kBins = 4096;
constexpr int kBinShift = 20;

__global__ void fill_u32_kernel(uint32_t* __restrict__ p, int64_t n, uint32_t v) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

__device__ __forceinline__ int row_vis(const TopkParams& p, int t) {
  return min(max(p.tok_vis[t], 0), p.max_vis);
}

__global__ __launch_bounds__(256) void topk_hist_kernel(TopkParams p) {
  __shared__ uint32_t h[kBins];
  const int t = blockIdx.y;
  const int vis = row_vis(p, t);
  if (vis <= p.k) return;
  const int s_begin = blockIdx.x * p.slice;
  if (s_begin >= vis) return;
  const int s_end = min(s_begin + p.slice, vis);
  for (int i = threadIdx.x; i < kBins; i += 256) h[i] = 0;
  __syncthreads();
  const float* row = p.scores + (int64_t)t * p.ld;
  // the whole slice (8 float4 per thread) is loaded before any is binned
  f32x4 v[8];
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const int s = s_begin + 4 * threadIdx.x + 1024 * b;
    v[b] = (s + 3 < s_end) ? *reinterpret_cast<const f32x4*>(row + s) : f32x4{0.f, 0.f, 0.f, 0.f};
    if (s + 3 >= s_end)
      for (int e = 0; e < 4; ++e) v[b][e] = (s + e < s_end) ? row[s + e] : 0.f;
  }
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const int s = s_begin + 4 * threadIdx.x + 1024 * b;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (s + e < s_end) atomicAdd(&h[order_key(v[b][e]) >> kBinShift], 1u);
  }
  __syncthreads();
  uint32_t* gh = p.hist + (int64_t)t * kBins;
  for (int i = threadIdx.x; i < kBins; i += 256)
    if (h[i]) atomicAdd(&gh[i], h[i]);
}

// Threshold bin of a row from its global histogram: the bin b with
// count(bins > b) < k <= count(bins >= b); returns b and need = k - count(> b).
// Called by all 256 threads of a workgroup; 16 bins per thread, suffix sums
// with wave shuffles and one LDS exchange.
__device__ __forceinline__ void threshold_bin(const uint32_t* __restrict__ gh, uint32_t k, int* out_bin,
                                              uint32_t* out_need) {
  __shared__ uint32_t wtot[4];
  __shared__ int s_bin;
  __shared__ uint32_t s_need;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t loc[16];
  uint32_t sum = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    loc[i] = gh[tid * 16 + i];
    sum += loc[i];
  }
  uint32_t suf = sum;  // inclusive suffix sum within the wave
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t o = __shfl_down(suf, off);
    if (lane + off < 64) suf += o;
  }
  if (lane == 0) wtot[wave] = suf;
  __syncthreads();
  for (int w = wave + 1; w < 4; ++w) suf += wtot[w];
  const uint32_t above = suf - sum;  // bins owned by higher threads
  if (above < k && suf >= k) {
    uint32_t acc = above;
    for (int i = 15; i >= 0; --i) {
      if (acc + loc[i] >= k) {
        s_bin = tid * 16 + i;
        s_need = k - acc;
        break;
      }
      acc += loc[i];
    }
  }
  __syncthreads();
  *out_bin = s_bin;
  *out_need = s_need;
}

constexpr int kFilterCap = 2048;  // candidates a filter workgroup keeps in LDS

// Keys above the threshold bin ("definite") and inside it ("candidates") are
// gathered in LDS, then copied out behind one global atomic per list.
__global__ __launch_bounds__(256) void topk_filter_kernel(TopkParams p) {
  __shared__ int l_def[DSA_MAX_TOPK];
  __shared__ uint32_t l_ck[kFilterCap];
  __shared__ int l_ci[kFilterCap];
  __shared__ int n_def, n_cand, n_cand2;
  __shared__ uint32_t base_def, base_cand;
  const int t = blockIdx.y;
  const int tid = threadIdx.x;
  const int vis = row_vis(p, t);
  if (vis <= p.k) return;
  const int s_begin = blockIdx.x * p.slice;
  if (s_begin >= vis) return;
  const int s_end = min(s_begin + p.slice, vis);
  uint32_t* ctr = p.ctr + (int64_t)t * 4;
  if (tid == 0) {
    n_def = 0;
    n_cand = 0;
    n_cand2 = 0;
  }
  int ibin;
  uint32_t need;
  threshold_bin(p.hist + (int64_t)t * kBins, (uint32_t)p.k, &ibin, &need);
  const uint32_t bin = (uint32_t)ibin;
  if (blockIdx.x == 0 && tid == 0) {
    ctr[2] = bin;
    ctr[3] = need;
  }
  const float* row = p.scores + (int64_t)t * p.ld;
  f32x4 v[8];
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const int s = s_begin + 4 * tid + 1024 * b;
    v[b] = (s + 3 < s_end) ? *reinterpret_cast<const f32x4*>(row + s) : f32x4{0.f, 0.f, 0.f, 0.f};
    if (s + 3 >= s_end)
      for (int e = 0; e < 4; ++e) v[b][e] = (s + e < s_end) ? row[s + e] : 0.f;
  }
  __syncthreads();  // counters initialised
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const int s = s_begin + 4 * tid + 1024 * b;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (s + e >= s_end) break;
      const uint32_t key = order_key(v[b][e]);
      const uint32_t d = key >> kBinShift;
      if (d > bin) {
        const int pos = atomicAdd(&n_def, 1);
        if (pos < DSA_MAX_TOPK) l_def[pos] = s + e;
      } else if (d == bin) {
        const int pos = atomicAdd(&n_cand, 1);
        if (pos < kFilterCap) {
          l_ck[pos] = key;
          l_ci[pos] = s + e;
        }
      }
    }
  }
  __syncthreads();
  if (tid == 0) {
    base_def = atomicAdd(&ctr[0], (uint32_t)n_def);
    base_cand = atomicAdd(&ctr[1], (uint32_t)n_cand);
  }
  __syncthreads();
  int32_t* defrow = p.defbuf + (int64_t)t * p.k;
  for (int i = tid; i < n_def; i += 256)
    if (base_def + i < (uint32_t)p.k) defrow[base_def + i] = l_def[i];
  uint32_t* candrow = p.cand + (int64_t)t * p.cand_cap * 2;
  const int nc = n_cand;
  if (nc <= kFilterCap) {
    for (int i = tid; i < nc; i += 256) {
      const uint32_t pos = base_cand + i;
      if (pos < (uint32_t)p.cand_cap) {
        candrow[2 * pos] = l_ck[i];
        candrow[2 * pos + 1] = (uint32_t)l_ci[i];
      }
    }
  } else {
    // more candidates than LDS holds: write them all straight from a rescan
    for (int s = s_begin + tid; s < s_end; s += 256) {
      const uint32_t key = order_key(row[s]);
      if ((key >> kBinShift) == bin) {
        const uint32_t pos = base_cand + (uint32_t)atomicAdd(&n_cand2, 1);
        if (pos < (uint32_t)p.cand_cap) {
          candrow[2 * pos] = key;
          candrow[2 * pos + 1] = (uint32_t)s;
        }
      }
    }
  }
}

__device__ __forceinline__ uint64_t composite(uint32_t key, uint32_t idx) {
  return ((uint64_t)(key & 0xFFFFFu) << 36) | ((uint64_t)(0xFFFFFFFFu - idx) << 4);
}

__device__ __forceinline__ int translate_one(int li, int r, const int32_t* __restrict__ bt, int bt_stride,
                                             int plog2) {
  if (li < 0) return -1;
  const int lp = li >> plog2;
  int pg;
  if (bt) {
    if (lp >= bt_stride) return -1;
    pg = bt[(int64_t)r * bt_stride + lp];
  } else {
    pg = r;
  }
  if (pg < 0) return -1;
  return (pg << plog2) | (li & ((1 << plog2) - 1));
}

constexpr int kFinalCap = 4096;  // candidates the finalize workgroup refines in LDS
constexpr int kWinIdx = 1024 * 8 * 32;  // indices per bitmap window (8 words per thread)

__global__ __launch_bounds__(1024) void topk_finalize_kernel(TopkParams p) {
  __shared__ int out[DSA_MAX_TOPK];
  __shared__ uint32_t cand_lds[2 * kFinalCap];  // candidate keys, candidate indices; later the bitmap
  uint32_t* ck = cand_lds;
  uint32_t* ci = cand_lds + kFinalCap;
  __shared__ uint32_t h[256];  // radix bins; later the 16 wave totals
  __shared__ uint32_t wsum[4];
  __shared__ uint64_t s_prefix;
  __shared__ int s_need, s_done, s_cnt;
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int vis = row_vis(p, t);
  const int K = min(p.k, vis);
  const int r = p.tok_req ? p.tok_req[t] : 0;
  int32_t* idx = p.idx + (int64_t)t * p.k;
  int32_t* rows = p.rows ? p.rows + (int64_t)t * p.k : nullptr;

  if (vis <= p.k) {
    for (int j = tid; j < p.k; j += blockDim.x) {
      const int li = j < vis ? j : -1;
      idx[j] = li;
      if (rows) rows[j] = translate_one(li, r, p.block_table, p.bt_stride, p.plog2);
    }
    if (p.count && tid == 0) p.count[t] = K;
    return;
  }

  const uint32_t* ctr = p.ctr + (int64_t)t * 4;
  const int ndef = (int)ctr[0];
  const int ncand = (int)ctr[1];
  const uint32_t bin = ctr[2];
  const uint32_t* candrow = p.cand + (int64_t)t * p.cand_cap * 2;
  const float* srow = p.scores + (int64_t)t * p.ld;
  // candidate source: LDS copy, the global candidate buffer, or the score row
  const int mode = (ncand <= kFinalCap) ? 0 : (ncand <= p.cand_cap ? 1 : 2);
  const int nsrc = mode == 2 ? vis : ncand;
  if (mode == 0)
    for (int i = tid; i < ncand; i += blockDim.x) {
      ck[i] = candrow[2 * i];
      ci[i] = candrow[2 * i + 1];
    }
  auto fetch = [&](int i, uint32_t& key, uint32_t& li) -> bool {
    if (mode == 0) {
      key = ck[i];
      li = ci[i];
      return true;
    }
    if (mode == 1) {
      key = candrow[2 * i];
      li = candrow[2 * i + 1];
      return true;
    }
    key = order_key(srow[i]);
    li = (uint32_t)i;
    return (key >> kBinShift) == bin;
  };

  if (tid == 0) {
    s_prefix = 0;
    s_need = (int)ctr[3];
    s_done = 0;
  }
  int shift = 48;
  for (;; shift -= 8) {
    if (tid < 256) h[tid] = 0;
    __syncthreads();
    const uint64_t prefix = s_prefix;
    const uint32_t need = (uint32_t)s_need;  // read by all before the update below
    for (int i = tid; i < nsrc; i += blockDim.x) {
      uint32_t key, li;
      if (!fetch(i, key, li)) continue;
      const uint64_t v = composite(key, li);
      if ((v >> (shift + 8)) == prefix) atomicAdd(&h[(v >> shift) & 255u], 1u);
    }
    __syncthreads();
    // suffix sums of the 256 bins: waves 0..3, one bin per lane
    uint32_t hv = 0, suf = 0;
    if (tid < 256) {
      hv = h[tid];
      suf = hv;
      const int lane = tid & 63;
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t o = __shfl_down(suf, off);
        if (lane + off < 64) suf += o;
      }
      if (lane == 0) wsum[tid >> 6] = suf;
    }
    __syncthreads();
    if (tid < 256) {
      for (int w = (tid >> 6) + 1; w < 4; ++w) suf += wsum[w];
      const uint32_t above = suf - hv;       // count in higher bins
      if (above < need && suf >= need) {     // exactly one bin qualifies
        const uint32_t nn = need - above;
        s_need = (int)nn;
        s_prefix = (prefix << 8) | (uint64_t)tid;
        s_done = (hv == nn) || shift == 0;
      }
    }
    __syncthreads();
    if (s_done) break;
  }
  const uint64_t thr = s_prefix;

  // winners: definite entries, then candidates at or above the threshold
  for (int i = tid; i < ndef; i += blockDim.x) out[i] = p.defbuf[(int64_t)t * p.k + i];
  if (tid == 0) s_cnt = ndef;
  __syncthreads();
  for (int i = tid; i < nsrc; i += blockDim.x) {
    uint32_t key, li;
    if (!fetch(i, key, li)) continue;
    if ((composite(key, li) >> shift) >= thr) {
      const int pos = atomicAdd(&s_cnt, 1);
      if (pos < DSA_MAX_TOPK) out[pos] = (int)li;
    }
  }
  __syncthreads();
  // order the K winners by index: mark them in an LDS bitmap window by window
  // (256K indices per window), then each thread emits the set bits of its 8
  // words at its prefix-sum offset
  uint32_t* bm = cand_lds;  // the candidate area (8192 words) is free now
  int emitted = 0;
  for (int w0 = 0; w0 < vis; w0 += kWinIdx) {
    for (int i = tid; i < kWinIdx / 32; i += blockDim.x) bm[i] = 0;
    __syncthreads();
    for (int i = tid; i < K; i += blockDim.x) {
      const int li = out[i] - w0;
      if (li >= 0 && li < kWinIdx) atomicOr(&bm[li >> 5], 1u << (li & 31));
    }
    __syncthreads();
    uint32_t words[8];
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      words[i] = bm[tid * 8 + i];
      cnt += __popc(words[i]);
    }
    // exclusive prefix over the 1024 threads: waves of 64, then 16 wave totals
    const int lane = tid & 63, wave = tid >> 6;
    int inc = cnt;
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(inc, off);
      if (lane >= off) inc += o;
    }
    if (lane == 63) h[wave] = (uint32_t)inc;
    __syncthreads();
    int before = emitted + inc - cnt;
    for (int w = 0; w < wave; ++w) before += (int)h[w];
    int tot = 0;
    for (int w = 0; w < 16; ++w) tot += (int)h[w];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t x = words[i];
      while (x) {
        const int b = __ffs(x) - 1;
        x &= x - 1;
        const int li = w0 + (tid * 8 + i) * 32 + b;
        idx[before] = li;
        if (rows) rows[before] = translate_one(li, r, p.block_table, p.bt_stride, p.plog2);
        ++before;
      }
    }
    emitted += tot;
    __syncthreads();
  }
  for (int j = K + tid; j < p.k; j += blockDim.x) {
    idx[j] = -1;
    if (rows) rows[j] = -1;
  }
  if (p.count && tid == 0) p.count[t] = K;
}

__global__ void translate_kernel(const int32_t* __restrict__ idx, int k, int T, const int32_t* __restrict__ tok_req,
                                 const int32_t* __restrict__ bt, int bt_stride, int plog2, int32_t* __restrict__ rows) {
  const int64_t n = (int64_t)T * k;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int t = (int)(i / k);
    rows[i] = translate_one(idx[i], tok_req[t], bt, bt_stride, plog2);
  }
}

dsa_status launch_topk(const TopkParams& p, hipStream_t stream) {
  // histograms and counters are contiguous in the workspace: one fill
  const int64_t nz = (int64_t)(p.ctr - p.hist) + (int64_t)p.T * 4;
  hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)std::min<int64_t>((nz + 255) / 256, 4096)), dim3(256), 0,
                     stream, p.hist, nz, 0u);
  dim3 grid(p.nslices, p.T);
  hipLaunchKernelGGL(topk_hist_kernel, grid, dim3(256), 0, stream, p);
  hipLaunchKernelGGL(topk_filter_kernel, grid, dim3(256), 0, stream, p);
  hipLaunchKernelGGL(topk_finalize_kernel, dim3(p.T), dim3(1024), 0, stream, p);
  return hipGetLastError() == hipSuccess ? DSA_OK : DSA_ERR_HIP;
}

dsa_status launch_translate(const int32_t* idx, int k, int T, const int32_t* tok_req, const int32_t* block_table,
                            int bt_stride, int plog2, int32_t* rows, hipStream_t stream) {
  const int64_t n = (int64_t)T * k;
  hipLaunchKernelGGL(translate_kernel, dim3((unsigned)std::min<int64_t>((n + 255) / 256, 8192)), dim3(256), 0,
                     stream, idx, k, T, tok_req, block_table, bt_stride, plog2, rows);
  return hipGetLastError() == hipSuccess ? DSA_OK : DSA_ERR_HIP;
}

}  // namespace dsa
