// Exact top-k merge across W context shards, emulated on one device.
//
// Kimi K3.1 Pro day-0 page, "Long context: decode context parallel" and
// "Exact top-k merge": shard r of W holds every W-th token (global s = j*W + r
// at local position j) and ranks only its own tokens.  Each shard sends its
// best few candidates with their scores, every receiver radix-selects the
// global top-k from the union, and a shard whose whole message was selected
// (so that it may hold more of the top-k than it sent) re-sends its full local
// top-k for that row, after which the row is selected again.  Candidates are
// 64-bit composites (order key of the fp32 score << 32 | ~global index): the
// larger composite ranks first, equal scores go to the lower index, and every
// composite of a row is distinct.
//
// Launch sequence (all on the caller's stream, no host round trip):
//   shard_vis     n_r(t) = ceil((vis_t - r) / W) for every (r, t)
//   local top-k   the per-row top-k on the W*T shard rows (k per row, the full
//                 local top-k a shard keeps for a possible re-send)
//   pack(1)       per shard row, the cand best of its local top-k -> exchange
//   merge(1)      per row: select K_t = min(k, vis_t) from the union; flag the
//                 shards that must re-send, or emit the ordered result
//   pack(2)       flagged shard rows: the full local top-k -> exchange
//   merge(2)      flagged rows: select again and emit (cannot flag again)
#include "common.h"
#include "kernels.h"

namespace dsa {

namespace {

constexpr int kMergeThreads = 1024;
constexpr int kMergePer = kMaxShards * DSA_MAX_TOPK / kMergeThreads;  // 32 composites per thread
constexpr int kPackThreads = 256;
constexpr int kPackPer = DSA_MAX_TOPK / kPackThreads;                   // 8

struct SelLds {
  uint32_t hist[256];
  uint32_t wsum[16];
  uint64_t prefix;
  int rho;
  int done;
};

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t o = __shfl_up(v, d, 64);
    if (lane >= d) v += o;
  }
  return v;
}

// The rho-th largest nonzero composite held by the block (PER per thread, 0 =
// empty slot), 1 <= rho <= number of nonzero composites.  Radix select over
// 8-bit digits from the top; stops at the first digit whose chosen bin is
// taken whole.  On return a composite c is among the rho largest iff
// c != 0 and (c >> shift) >= (prefix >> shift).
template <int PER>
__device__ void select_rank(const uint64_t (&c)[PER], int rho, SelLds& L, uint64_t& out_prefix, int& out_shift) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint64_t prefix = 0;
  int shift = 56;
  for (int pass = 0; pass < 8; ++pass, shift -= 8) {
    for (int b = tid; b < 256; b += blockDim.x) L.hist[b] = 0;
    __syncthreads();
    const uint64_t hi_mask = pass == 0 ? 0ull : (~0ull << (shift + 8));
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (c[i] != 0 && ((c[i] ^ prefix) & hi_mask) == 0) atomicAdd(&L.hist[(uint32_t)(c[i] >> shift) & 255u], 1u);
    }
    __syncthreads();
    // inclusive scan over bins in descending order: thread j holds bin 255 - j
    const uint32_t h = tid < 256 ? L.hist[255 - tid] : 0u;
    uint32_t incl = wave_incl_scan(h);
    if (lane == 63 && wave < 4) L.wsum[wave] = incl;
    __syncthreads();
    if (tid < 256) {
      for (int w = 0; w < wave; ++w) incl += L.wsum[w];
      const uint32_t above = incl - h;
      if (above < (uint32_t)rho && incl >= (uint32_t)rho) {
        const int r2 = rho - (int)above;
        L.prefix = prefix | ((uint64_t)(255 - tid) << shift);
        L.rho = r2;
        L.done = (int)h == r2;
      }
    }
    __syncthreads();
    prefix = L.prefix;
    rho = L.rho;
    const int done = L.done;
    if (done) break;
  }
  // (distinct composites end the loop by the last digit at the latest)
  out_prefix = prefix;
  out_shift = max(shift, 0);
}

__device__ __forceinline__ bool selected(uint64_t c, uint64_t prefix, int shift) {
  return c != 0 && (c >> shift) >= (prefix >> shift);
}

__device__ __forceinline__ int shard_count(int vis, int r, int W) {
  return vis > r ? (vis - r + W - 1) / W : 0;
}

__device__ __forceinline__ int clamp_vis(const MergeParams& p, int t) {
  return min(max(p.tok_vis[t], 0), p.max_vis);
}

__global__ __launch_bounds__(256) void shard_vis_kernel(MergeParams p) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= p.W * p.T) return;
  const int r = i / p.T, t = i - r * p.T;
  p.lvis[i] = shard_count(clamp_vis(p, t), r, p.W);
}

// One workgroup per shard row (r, t): its local top-k (ascending local
// positions) -> composites; round 1 sends the cand best of them, round 2 (only
// for flagged shard rows) sends them all.
__global__ __launch_bounds__(kPackThreads) void pack_kernel(MergeParams p, int round) {
  __shared__ SelLds L;
  __shared__ int s_slot;
  const int sr = blockIdx.x;  // r * T + t
  const int r = sr / p.T, t = sr - r * p.T;
  const int tid = threadIdx.x;
  if (round == 2 && p.flags[t * p.W + r] == 0) return;
  const int m = min(p.k, p.lvis[sr]);
  const int32_t* lidx = p.lidx + (int64_t)sr * p.k;
  const float* row = p.scores + (int64_t)sr * p.ld;
  uint64_t c[kPackPer];
#pragma unroll
  for (int i = 0; i < kPackPer; ++i) {
    const int e = tid + kPackThreads * i;
    c[i] = 0;
    if (e < m) {
      const int j = lidx[e];
      const uint32_t g = (uint32_t)j * (uint32_t)p.W + (uint32_t)r;
      c[i] = ((uint64_t)order_key(row[j]) << 32) | (uint64_t)(~g);
    }
  }
  uint64_t* out = p.xbuf + (int64_t)sr * p.k;
  const int send = round == 1 ? min(p.cand, m) : m;
  if (send == m) {
#pragma unroll
    for (int i = 0; i < kPackPer; ++i) {
      const int e = tid + kPackThreads * i;
      if (e < m) out[e] = c[i];
    }
  } else {
    uint64_t prefix;
    int shift;
    select_rank<kPackPer>(c, send, L, prefix, shift);
    if (tid == 0) s_slot = 0;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kPackPer; ++i) {
      if (selected(c[i], prefix, shift)) {
        const int slot = atomicAdd(&s_slot, 1);
        if (slot < send) out[slot] = c[i];
      }
    }
  }
  if (tid == 0) p.xcnt[sr] = send;
}

// One workgroup per query row: select from the union of the shards' messages,
// decide the re-sends (round 1), emit the ascending global indices.
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(MergeParams p, int round) {
  __shared__ SelLds L;
  __shared__ int s_pre[kMaxShards + 1];
  __shared__ int s_sel[kMaxShards];
  __shared__ int s_any;
  __shared__ int s_slot;
  __shared__ uint32_t s_out[DSA_MAX_TOPK];
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int W = p.W;
  if (round == 2 && p.rowflag[t] == 0) return;
  const int vis = clamp_vis(p, t);
  const int K = min(p.k, vis);
  int32_t* idx = p.idx + (int64_t)t * p.k;
  if (tid == 0) {
    int acc = 0;
    for (int r = 0; r < W; ++r) {
      s_pre[r] = acc;
      acc += p.xcnt[r * p.T + t];
      s_sel[r] = 0;
    }
    s_pre[W] = acc;
    s_any = 0;
    s_slot = 0;
  }
  __syncthreads();
  const int ntot = s_pre[W];

  uint64_t c[kMergePer];
#pragma unroll
  for (int i = 0; i < kMergePer; ++i) {
    const int e = tid + kMergeThreads * i;
    c[i] = 0;
    if (e < ntot) {
      int r = 0;
      while (r + 1 < W && s_pre[r + 1] <= e) ++r;
      c[i] = p.xbuf[(int64_t)(r * p.T + t) * p.k + (e - s_pre[r])];
    }
  }
  uint64_t prefix = 0;
  int shift = 0;
  if (K > 0 && ntot > K) select_rank<kMergePer>(c, K, L, prefix, shift);
  // (ntot <= K: every composite is selected; prefix 0 / shift 0 admits all)

#pragma unroll
  for (int i = 0; i < kMergePer; ++i) {
    if (K > 0 && selected(c[i], prefix, shift)) {
      const uint32_t g = ~(uint32_t)c[i];
      atomicAdd(&s_sel[g % (uint32_t)W], 1);
    }
  }
  __syncthreads();
  if (round == 1 && tid < W) {
    const int r = tid;
    const int n = shard_count(vis, r, W);
    const int sent = s_pre[r + 1] - s_pre[r];
    const int flag = (K > 0 && s_sel[r] == sent && sent < min(p.k, n)) ? 1 : 0;
    p.flags[t * W + r] = flag;
    if (flag) atomicOr(&s_any, 1);
  }
  __syncthreads();
  if (round == 1) {
    if (tid == 0) p.rowflag[t] = s_any;
    if (s_any) return;  // emitted by round 2
  }

  // ascending global indices: gather the winners, bitonic sort in LDS
  int n2 = 1;
  while (n2 < K) n2 <<= 1;
  for (int j = tid; j < n2; j += kMergeThreads) s_out[j] = 0xFFFFFFFFu;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kMergePer; ++i) {
    if (K > 0 && selected(c[i], prefix, shift)) {
      const int slot = atomicAdd(&s_slot, 1);
      if (slot < n2) s_out[slot] = ~(uint32_t)c[i];
    }
  }
  __syncthreads();
  for (int size = 2; size <= n2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < (n2 >> 1); i += kMergeThreads) {
        const int lo = ((i & ~(stride - 1)) << 1) | (i & (stride - 1));
        const int hi = lo + stride;
        const bool up = (lo & size) == 0;
        const uint32_t a = s_out[lo], b = s_out[hi];
        if ((a > b) == up) {
          s_out[lo] = b;
          s_out[hi] = a;
        }
      }
      __syncthreads();
    }
  }
  for (int j = tid; j < p.k; j += kMergeThreads) idx[j] = j < K ? (int32_t)s_out[j] : -1;
  if (p.count && tid == 0) p.count[t] = K;
}

}  // namespace

dsa_status launch_topk_sharded(const MergeParams& p, const TopkParams& local, hipStream_t stream) {
  const int n = p.W * p.T;
  hipLaunchKernelGGL(shard_vis_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, p);
  if (hipGetLastError() != hipSuccess) return DSA_ERR_HIP;
  dsa_status st = launch_topk(local, stream);
  if (st != DSA_OK) return st;
  hipLaunchKernelGGL(pack_kernel, dim3(n), dim3(kPackThreads), 0, stream, p, 1);
  hipLaunchKernelGGL(merge_kernel, dim3(p.T), dim3(kMergeThreads), 0, stream, p, 1);
  hipLaunchKernelGGL(pack_kernel, dim3(n), dim3(kPackThreads), 0, stream, p, 2);
  hipLaunchKernelGGL(merge_kernel, dim3(p.T), dim3(kMergeThreads), 0, stream, p, 2);
  return hipGetLastError() == hipSuccess ? DSA_OK : DSA_ERR_HIP;
}

}  // namespace dsa
