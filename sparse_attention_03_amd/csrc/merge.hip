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
//   top-k(cand)   every shard row selects its cand best local positions (the
//                 per-row top-k kernels on the W*T shard rows)
//   pack(1)       -> composites in the exchange buffer
//   merge(1)      per row: select K_t = min(k, vis_t) from the union; flag the
//                 shards that must re-send, or emit the ordered result
//   top-k(k)      flagged shard rows select their full local top-k (the other
//                 shard rows see no visible token and return at once)
//   pack(2)       flagged shard rows -> exchange
//   merge(2)      flagged rows: select again and emit (cannot flag again)
#include "common.h"
#include "kernels.h"
#include "radix.h"

namespace dsa {

namespace {

constexpr int kMergeThreads = 1024;
constexpr int kMergeLdsCap = 4096;  // unions up to this many composites are staged in LDS
constexpr int kPackThreads = 256;

__device__ __forceinline__ bool selected(uint64_t c, uint64_t prefix, int hi) {
  return c != 0 && shr_sat<uint64_t>(c, hi) >= shr_sat<uint64_t>(prefix, hi);
}

__device__ __forceinline__ int shard_count(int vis, int r, int W) {
  return vis > r ? (vis - r + W - 1) / W : 0;
}

__device__ __forceinline__ int row_vis(const MergeParams& p, int t) {
  return clamp_vis(p.tok_vis[t], p.max_vis);
}

__global__ __launch_bounds__(256) void shard_vis_kernel(MergeParams p) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= p.W * p.T) return;
  const int r = i / p.T, t = i - r * p.T;
  p.lvis[i] = shard_count(row_vis(p, t), r, p.W);
}

// One workgroup per shard row (r, t): the shard's selected local positions
// (ascending, `kk` per row: cand in the first exchange, k in the re-send)
// -> composites in the exchange buffer.  The re-send packs only the flagged
// shard rows.
__global__ __launch_bounds__(kPackThreads) void pack_kernel(MergeParams p, int phase) {
  const int sr = blockIdx.x;  // r * T + t
  const int r = sr / p.T, t = sr - r * p.T;
  const int tid = threadIdx.x;
  if (phase == 2 && p.flags[t * p.W + r] == 0) return;
  const int kk = phase == 1 ? p.cand : p.k;
  const int m = min(kk, phase == 1 ? p.lvis[sr] : p.lvis2[sr]);
  const int32_t* lidx = p.lidx + (int64_t)sr * kk;
  const float* row = p.scores + (int64_t)sr * p.ld;
  uint64_t* out = p.xbuf + (int64_t)sr * p.k;
  for (int e = tid; e < m; e += kPackThreads) {
    const int j = lidx[e];
    const uint32_t g = (uint32_t)j * (uint32_t)p.W + (uint32_t)r;
    out[e] = ((uint64_t)order_key(row[j]) << 32) | (uint64_t)(~g);
  }
  if (tid == 0) p.xcnt[sr] = m;
}

// One workgroup per query row: select from the union of the shards' messages,
// decide the re-sends (first exchange), emit the ascending global indices.
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(MergeParams p, int phase) {
  __shared__ RadixLds<uint64_t, kMergeThreads> L;
  __shared__ int s_pre[kMaxShards + 1];
  __shared__ int s_sel[kMaxShards];
  __shared__ int s_any;
  __shared__ int s_slot;
  __shared__ __align__(16) uint32_t s_out[DSA_MAX_TOPK];
  __shared__ __align__(16) uint32_t s_out2[DSA_MAX_TOPK];
  __shared__ uint64_t s_comp[kMergeLdsCap];
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int W = p.W;
  if (phase == 2 && p.rowflag[t] == 0) return;
  const int vis = row_vis(p, t);
  const int K = min(p.k, vis);
  int32_t* idx = p.idx + (int64_t)t * p.k;
  if (tid < W) {
    s_pre[tid + 1] = p.xcnt[tid * p.T + t];  // loads in parallel, summed below
    s_sel[tid] = 0;
  }
  if (tid == 0) {
    s_pre[0] = 0;
    s_any = 0;
    s_slot = 0;
  }
  __syncthreads();
  if (tid < 64) {  // inclusive scan of the counts by the first wave (W <= 16)
    const uint32_t v = tid < W ? (uint32_t)s_pre[tid + 1] : 0u;
    const uint32_t inc = wave_incl_scan32(v);
    if (tid < W) s_pre[tid + 1] = (int)inc;
  }
  __syncthreads();
  const int ntot = s_pre[W];
  // shard starts in registers: an element's shard is the number of starts
  // at or below it (independent compares, no dependent LDS reads)
  int pre[kMaxShards];
#pragma unroll
  for (int q = 0; q < kMaxShards; ++q) pre[q] = q < W ? s_pre[q] : 0x7fffffff;

  // the union: staged in LDS when it fits, else read from the exchange buffer
  // (L2-resident) on every pass
  auto comp_at = [&](int e) {
    int r = -1, base = 0;
#pragma unroll
    for (int q = 0; q < kMaxShards; ++q) {
      if (pre[q] <= e) {
        r = q;
        base = pre[q];
      }
    }
    return p.xbuf[(int64_t)(r * p.T + t) * p.k + (e - base)];
  };
  const bool staged = ntot <= kMergeLdsCap;
  if (staged) {
    for (int e = tid; e < ntot; e += kMergeThreads) s_comp[e] = comp_at(e);
    __syncthreads();
  }
  auto each = [&](auto f) {
    if (staged) {
      for (int e = tid; e < ntot; e += kMergeThreads) f(s_comp[e]);
    } else {
      for (int e = tid; e < ntot; e += kMergeThreads) f(comp_at(e));
    }
  };
  uint64_t prefix = 0;
  int shift = 0;
  if (K > 0 && ntot > K) {
    int rho_eq;  // composites are distinct: the last digit is always taken whole
    radix_kth<uint64_t, kMergeThreads>(each, K, L, prefix, shift, rho_eq);
  }
  // (ntot <= K: every composite is selected; prefix 0 / shift 0 admits all)

  if (K > 0) {
    each([&](uint64_t c) {
      if (selected(c, prefix, shift)) atomicAdd(&s_sel[(~(uint32_t)c) % (uint32_t)W], 1);
    });
  }
  __syncthreads();
  if (phase == 1 && tid < W) {
    const int r = tid;
    const int n = shard_count(vis, r, W);
    const int sent = s_pre[r + 1] - s_pre[r];
    const int flag = (K > 0 && s_sel[r] == sent && sent < min(p.k, n)) ? 1 : 0;
    p.flags[t * W + r] = flag;
    p.lvis2[r * p.T + t] = flag ? n : 0;  // the shards that select their full local top-k
    if (flag) atomicOr(&s_any, 1);
  }
  __syncthreads();
  if (phase == 1) {
    if (tid == 0) p.rowflag[t] = s_any;
    if (s_any) return;  // emitted after the re-send
  }

  // ascending global indices: gather the winners into 2048 slots (padding
  // 0xFFFFFFFF sorts last), then a bitonic sort with two slots per thread:
  // partners within a wave exchange by lane shuffles, partners in other waves
  // through LDS (two buffers used in turn, one barrier per such stage)
  for (int j = tid; j < DSA_MAX_TOPK; j += kMergeThreads) s_out[j] = 0xFFFFFFFFu;
  __syncthreads();
  if (K > 0) {
    each([&](uint64_t c) {
      if (selected(c, prefix, shift)) {
        const int slot = atomicAdd(&s_slot, 1);
        if (slot < DSA_MAX_TOPK) s_out[slot] = ~(uint32_t)c;
      }
    });
  }
  __syncthreads();
  const uint2 ab = reinterpret_cast<const uint2*>(s_out)[tid];  // slots 2*tid, 2*tid + 1
  uint32_t a = ab.x, b = ab.y;
  int cur = 1;
#pragma unroll
  for (int size = 2; size <= DSA_MAX_TOPK; size <<= 1) {
    const bool up = ((2 * tid) & size) == 0;
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      if (stride == 1) {
        if ((a > b) == up) {
          const uint32_t x = a;
          a = b;
          b = x;
        }
        continue;
      }
      const int m = stride >> 1;  // partner thread tid ^ m holds the partner slots
      uint32_t pa, pb;
      if (m < 64) {
        pa = lane_xor(a, m);
        pb = lane_xor(b, m);
      } else {
        uint2* bp = reinterpret_cast<uint2*>(cur ? s_out2 : s_out);
        bp[tid] = make_uint2(a, b);
        __syncthreads();
        const uint2 q = bp[tid ^ m];
        pa = q.x;
        pb = q.y;
        cur ^= 1;
      }
      const bool keep_min = ((tid & m) == 0) == up;
      a = keep_min ? min(a, pa) : max(a, pa);
      b = keep_min ? min(b, pb) : max(b, pb);
    }
  }
  if (2 * tid < p.k) idx[2 * tid] = 2 * tid < K ? (int32_t)a : -1;
  if (2 * tid + 1 < p.k) idx[2 * tid + 1] = 2 * tid + 1 < K ? (int32_t)b : -1;
  if (p.count && tid == 0) p.count[t] = K;
}

}  // namespace

dsa_status launch_topk_sharded(const MergeParams& p, const TopkParams& local, hipStream_t stream) {
  const int n = p.W * p.T;
  hipLaunchKernelGGL(shard_vis_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, p);
  if (hipGetLastError() != hipSuccess) return DSA_ERR_HIP;
  // first exchange: every shard row selects its cand best positions
  TopkParams l1 = local;
  l1.tok_vis = p.lvis;
  l1.k = p.cand;
  dsa_status st = launch_topk(l1, stream);
  if (st != DSA_OK) return st;
  hipLaunchKernelGGL(pack_kernel, dim3(n), dim3(kPackThreads), 0, stream, p, 1);
  hipLaunchKernelGGL(merge_kernel, dim3(p.T), dim3(kMergeThreads), 0, stream, p, 1);
  // re-send: flagged shard rows select their full local top-k (every other
  // shard row has lvis2 = 0 and its workgroups return at once)
  TopkParams l2 = local;
  l2.tok_vis = p.lvis2;
  l2.k = p.k;
  st = launch_topk(l2, stream);
  if (st != DSA_OK) return st;
  hipLaunchKernelGGL(pack_kernel, dim3(n), dim3(kPackThreads), 0, stream, p, 2);
  hipLaunchKernelGGL(merge_kernel, dim3(p.T), dim3(kMergeThreads), 0, stream, p, 2);
  return hipGetLastError() == hipSuccess ? DSA_OK : DSA_ERR_HIP;
}

DSA_DEBUG_TAKE(merge)

}  // namespace dsa
