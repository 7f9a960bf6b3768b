// MSA block-sparse decode (MiniMax M3.1 page, "MSA primer"; its AMD section
// for the FP8/NVFP4 caches): 128-token blocks, one index query per GQA group
// scored against one shared FP8 index-key head, a max-pool to one score per
// block, the top blocks (the most recent always kept), and exact attention of
// every query head of a group over its group's selected blocks.
//
//   msa_index_kernel   one workgroup per (request, block): the block's 128
//                      index keys are read once for every row and group of
//                      the request; scores on v_mfma_f32_16x16x32_bf16 with
//                      keys as M (FP8 -> BF16 is exact) and (row, group)
//                      queries as N; the block maximum over visible keys.
//   msa_select_kernel  one workgroup per (row, group): the most recent block
//                      plus the top - 1 best others, by a block radix select
//                      over (score order key, inverted block id) composites;
//                      ascending ids, -1 padded.
//   msa_attn_kernel    one 8-wave workgroup per (row, group): each wave runs
//                      its selected blocks in 16-key tiles -- S^T = K . Q^T
//                      (keys x heads, so the softmax weights land where the
//                      PV product wants its A operand), online softmax per
//                      head, O += P . V with V staged as BF16 rows in LDS and
//                      read transposed (ds_read_b64_tr_b16) -- then the waves'
//                      partial results merge by log-sum-exp.
#include "common.h"
#include "kernels.h"
#include "radix.h"

namespace dsa {

namespace {

constexpr int kBlk = 128;       // tokens per block
constexpr int kD = 128;         // head dim
constexpr int kAttnWaves = 8;
constexpr int kAttnSplits = kMsaSplits;  // workgroups per (row, group)
constexpr int kVStride = 136;   // bf16 per LDS V row (272 B)

__device__ __forceinline__ int msa_vis(const MsaParams& p, int t) { return clamp_vis(p.tok_vis[t], p.max_vis); }

__device__ __forceinline__ int msa_page(const MsaParams& p, int r, int b) {
  DSA_DEBUG_NOTE(b >= p.bt_stride, DSA_DEBUG_ROW_OUTSIDE);
  if (r < 0 || b < 0 || b >= p.bt_stride) return -1;
  const int pg = p.bt[(int64_t)r * p.bt_stride + b];
  DSA_DEBUG_NOTE(pg < 0 || pg >= p.pool_blocks, DSA_DEBUG_ABSENT_PAGE);
  return (pg >= 0 && pg < p.pool_blocks) ? pg : -1;
}

constexpr int kIdxBlocks = 4;  // blocks per index workgroup

// 32 contiguous key bytes per lane (dims 32g .. 32g+31 of keys 32w + 16mt + c):
// k-step ks takes dims 32g + 8ks .. +8 from lane group g (any split of the 128
// dims works when the query side uses the same one).
struct KeyRegs {
  i32x4 v[2][2];
};

__device__ __forceinline__ void load_keys(const MsaParams& p, int page, int w, int g, int c, KeyRegs& k) {
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    if (page >= 0) {
      const i32x4* src = reinterpret_cast<const i32x4*>(p.idx_pool + (int64_t)page * (kBlk * kD) +
                                                        (32 * w + 16 * mt + c) * kD + 32 * g);
      k.v[mt][0] = __builtin_nontemporal_load(src);
      k.v[mt][1] = __builtin_nontemporal_load(src + 1);
    } else {
      k.v[mt][0] = i32x4{0, 0, 0, 0};
      k.v[mt][1] = i32x4{0, 0, 0, 0};
    }
  }
}

// One workgroup per (request, kIdxBlocks consecutive blocks): every wave
// scores 32 keys of each block for every (row, group) query of the request
// (keys as MFMA M, FP8 -> BF16 exact, queries as N), the next block's keys
// loading while the current one is scored; the per-wave block maxima meet in
// LDS once per query tile.
__global__ __launch_bounds__(256) void msa_index_kernel(MsaParams p) {
  __shared__ float red[kIdxBlocks][4][16];
  const int bb0 = blockIdx.x * kIdxBlocks, r = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, c = lane & 15;
  const int rs = p.req_row_start[r], nrows = p.req_row_start[r + 1] - rs;
  int vmax = 0;
  for (int i = 0; i < nrows; ++i) vmax = max(vmax, msa_vis(p, rs + i));
  const int nblk = min(kIdxBlocks, (vmax + kBlk - 1) / kBlk - bb0);
  if (nblk <= 0) return;
  const int nq = nrows * p.hkv;
  for (int q0 = 0; q0 < nq; q0 += 16) {
    const int qq = q0 + c;  // this lane's query column
    const bool qok = qq < nq;
    const int row = rs + (qok ? qq / p.hkv : 0), grp = qok ? qq % p.hkv : 0;
    const int vis = qok ? msa_vis(p, row) : 0;
    bf16x8 bq[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bq[ks] = bf16x8{};
      if (qok) bq[ks] = *reinterpret_cast<const bf16x8*>(p.q_idx + ((int64_t)row * p.hkv + grp) * kD + 32 * g + 8 * ks);
    }
    KeyRegs cur, nxt;
    int page = msa_page(p, r, bb0);
    load_keys(p, page, w, g, c, cur);
    for (int i = 0; i < nblk; ++i) {
      const int b = bb0 + i;
      const int npage = i + 1 < nblk ? msa_page(p, r, b + 1) : -1;
      if (i + 1 < nblk) load_keys(p, npage, w, g, c, nxt);
      f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        acc[mt] = mfma16x16x32(e4m3x8_to_bf16x8(cur.v[mt][0][0], cur.v[mt][0][1]), bq[0], acc[mt]);
        acc[mt] = mfma16x16x32(e4m3x8_to_bf16x8(cur.v[mt][0][2], cur.v[mt][0][3]), bq[1], acc[mt]);
        acc[mt] = mfma16x16x32(e4m3x8_to_bf16x8(cur.v[mt][1][0], cur.v[mt][1][1]), bq[2], acc[mt]);
        acc[mt] = mfma16x16x32(e4m3x8_to_bf16x8(cur.v[mt][1][2], cur.v[mt][1][3]), bq[3], acc[mt]);
      }
      float mx = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int tok = b * kBlk + 32 * w + 16 * mt + 4 * g + j;
          if (page >= 0 && tok < vis) mx = fmaxf(mx, acc[mt][j]);
        }
      mx = fmaxf(mx, __uint_as_float(lane_xor(__float_as_uint(mx), 16)));
      mx = fmaxf(mx, __uint_as_float(lane_xor(__float_as_uint(mx), 32)));
      if (lane < 16) red[i][w][lane] = mx;
      cur = nxt;
      page = npage;
    }
    __syncthreads();
    if (tid < 16 * kIdxBlocks) {
      const int i = tid >> 4, col = tid & 15;
      const int qc = q0 + col;
      const int b = bb0 + i;
      if (i < nblk && qc < nq) {
        const int rw = rs + qc / p.hkv, gp = qc % p.hkv;
        if (b * kBlk < msa_vis(p, rw)) {
          const float m = fmaxf(fmaxf(red[i][0][col], red[i][1][col]), fmaxf(red[i][2][col], red[i][3][col]));
          p.bscore[((int64_t)rw * p.hkv + gp) * p.nblk_ld + b] = m;
        }
      }
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void msa_select_kernel(MsaParams p) {
  __shared__ RadixLds<uint64_t, 256> L;
  __shared__ int s_sel[16];
  __shared__ int s_n;
  const int tg = blockIdx.x, t = tg / p.hkv;
  const int tid = threadIdx.x;
  const int vis = msa_vis(p, t);
  const int nb = (vis + kBlk - 1) / kBlk;
  int32_t* out = p.sel + (int64_t)tg * p.top;
  if (p.top == 1 && nb > 1) {  // only the most recent block
    if (tid == 0) out[0] = nb - 1;
    return;
  }
  if (nb <= p.top) {
    for (int j = tid; j < p.top; j += 256) out[j] = j < nb ? j : -1;
    return;
  }
  const float* bs = p.bscore + (int64_t)tg * p.nblk_ld;
  const int nother = nb - 1;
  auto each = [&](auto f) {
    for (int b = tid; b < nother; b += 256) f(((uint64_t)order_key(bs[b]) << 32) | (uint64_t)(~(uint32_t)b));
  };
  uint64_t prefix;
  int hi, rho;
  radix_kth<uint64_t, 256>(each, p.top - 1, L, prefix, hi, rho);
  if (tid == 0) s_n = 0;
  __syncthreads();
  each([&](uint64_t cc) {
    if (shr_sat<uint64_t>(cc, hi) >= shr_sat<uint64_t>(prefix, hi)) {
      const int slot = atomicAdd(&s_n, 1);
      if (slot < 15) s_sel[slot] = (int)(~(uint32_t)cc);
    }
  });
  __syncthreads();
  // the most recent block joins the winners; every id's output slot is its
  // rank among them (ids are distinct), one thread per id
  const int n = min(s_n, p.top - 1) + 1;
  if (tid == 0) s_sel[n - 1] = nb - 1;
  __syncthreads();
  if (tid < n) {
    const int v = s_sel[tid];
    int rank = 0;
    for (int i = 0; i < n; ++i) rank += s_sel[i] < v;
    out[rank] = v;
  } else if (tid < p.top) {
    out[tid] = -1;
  }
}

__global__ __launch_bounds__(64 * kAttnWaves) void msa_attn_kernel(MsaParams p) {
  __shared__ __align__(16) __bf16 vt[kAttnWaves][16 * kVStride];
  __shared__ float pm[kAttnWaves][16], pl[kAttnWaves][16];
  __shared__ float po[kAttnWaves][16][kD];
  const int tg = blockIdx.x, t = tg / p.hkv, grp = tg - t * p.hkv;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, c = lane & 15;
  // a row whose tok_req names no request reads no block
  const int r_raw = p.tok_req[t];
  DSA_DEBUG_NOTE(r_raw < 0 || r_raw >= p.R, DSA_DEBUG_REQ_OUTSIDE);
  const int r = (r_raw >= 0 && r_raw < p.R) ? r_raw : -1;
  const int vis = msa_vis(p, t);
  const int hbase = grp * p.G;
  const float lscale = p.sm_scale * p.k_scale;
  const int64_t tok_bytes = 2LL * p.hkv * kD;
  const int64_t page_bytes = (int64_t)kBlk * tok_bytes;
  // Q^T fragments: head c of the group, dims 32g + 8ks .. +8 (zero past G)
  bf16x8 bq[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    bq[ks] = bf16x8{};
    if (c < p.G) bq[ks] = *reinterpret_cast<const bf16x8*>(p.q + ((int64_t)t * p.hq + hbase + c) * kD + 32 * g + 8 * ks);
  }
  f32x4 O[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) O[u] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_c = -INFINITY, l_c = 0.f;  // running max / sum of head c
  __bf16* vrow = vt[w];
  const __bf16* vsrc = vrow + (4 * g + (c >> 2)) * kVStride + 4 * (c & 3);
  // split s of kAttnSplits takes selected blocks s*kAttnWaves + w, + kAttnWaves*kAttnSplits, ...
  const int split = blockIdx.y;
  for (int sj = split * kAttnWaves + w; sj < p.top; sj += kAttnWaves * kAttnSplits) {
    const int blk = p.sel[(int64_t)tg * p.top + sj];
    if (blk < 0) continue;
    const int page = msa_page(p, r, blk);
    if (page < 0) continue;
    const uint8_t* base = p.kv_pool + (int64_t)page * page_bytes + grp * kD;
    for (int tile = 0; tile < kBlk / 16; ++tile) {
      const int key0 = blk * kBlk + 16 * tile;
      if (key0 >= vis) break;
      // S^T[key 4g+i][head c] over the tile's 16 keys
      // (k-step ks takes dims 32g + 8ks .. +8 from lane group g, as the
      // query fragments do: 32 contiguous key bytes per lane)
      f32x4 s = {0.f, 0.f, 0.f, 0.f};
      const uint8_t* krow = base + (int64_t)(16 * tile + c) * tok_bytes;
      const i32x4 k0 = *reinterpret_cast<const i32x4*>(krow + 32 * g);
      const i32x4 k1 = *reinterpret_cast<const i32x4*>(krow + 32 * g + 16);
      s = mfma16x16x32(e4m3x8_to_bf16x8(k0[0], k0[1]), bq[0], s);
      s = mfma16x16x32(e4m3x8_to_bf16x8(k0[2], k0[3]), bq[1], s);
      s = mfma16x16x32(e4m3x8_to_bf16x8(k1[0], k1[1]), bq[2], s);
      s = mfma16x16x32(e4m3x8_to_bf16x8(k1[2], k1[3]), bq[3], s);
      // V rows of the tile -> BF16 in LDS (zero rows past vis)
      {
        const bool vok = key0 + c < vis;
        const uint4* vp = reinterpret_cast<const uint4*>(krow + p.hkv * kD + 32 * g);
        uint4 v0 = make_uint4(0u, 0u, 0u, 0u), v1 = v0;
        if (vok) {
          v0 = vp[0];
          v1 = vp[1];
        }
        bf16x8* dst = reinterpret_cast<bf16x8*>(vrow + c * kVStride + 32 * g);
        dst[0] = e4m3x8_to_bf16x8(v0.x, v0.y);
        dst[1] = e4m3x8_to_bf16x8(v0.z, v0.w);
        dst[2] = e4m3x8_to_bf16x8(v1.x, v1.y);
        dst[3] = e4m3x8_to_bf16x8(v1.z, v1.w);
      }
      float x[4];
      float tmax = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = key0 + 4 * g + i < vis;
        x[i] = ok ? s[i] * lscale : -INFINITY;
        tmax = fmaxf(tmax, x[i]);
      }
      tmax = fmaxf(tmax, __uint_as_float(lane_xor(__float_as_uint(tmax), 16)));
      tmax = fmaxf(tmax, __uint_as_float(lane_xor(__float_as_uint(tmax), 32)));
      const float m_new = fmaxf(m_c, tmax);  // finite: key0 < vis
      const float alpha = __expf(m_c - m_new);
      float pv[4], ps = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pv[i] = __expf(x[i] - m_new);
        ps += pv[i];
      }
      ps += __uint_as_float(lane_xor(__float_as_uint(ps), 16));
      ps += __uint_as_float(lane_xor(__float_as_uint(ps), 32));
      l_c = l_c * alpha + ps;
      m_c = m_new;
      // rescale the output rows (heads 4g+i): alpha of head h sits in lane h
      float ar[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) ar[i] = __shfl(alpha, 4 * g + i, 64);
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) O[u][i] *= ar[i];
      bf16x4 pa;
      pa[0] = (__bf16)pv[0];
      pa[1] = (__bf16)pv[1];
      pa[2] = (__bf16)pv[2];
      pa[3] = (__bf16)pv[3];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        typedef short s16x4 __attribute__((ext_vector_type(4)));
        const auto* src = (const __attribute__((address_space(3))) s16x4*)(const void*)(vsrc + 16 * u);
        const s16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16(const_cast<__attribute__((address_space(3))) s16x4*>(src));
        O[u] = mfma16x16x16(pa, __builtin_bit_cast(bf16x4, vb), O[u]);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  }
  // the wave's partial result
  if (g == 0) {
    pm[w][c] = m_c;
    pl[w][c] = l_c;
  }
#pragma unroll
  for (int u = 0; u < 8; ++u)
#pragma unroll
    for (int i = 0; i < 4; ++i) po[w][4 * g + i][16 * u + c] = O[u][i];
  __syncthreads();
  // the workgroup's partial (max, sum, unnormalised output) per head
  float* part = p.part + ((int64_t)tg * kAttnSplits + split) * kMsaPartFloats;
  for (int e = tid; e < 16 * kD; e += 64 * kAttnWaves) {
    const int h = e / kD, d = e - h * kD;
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < kAttnWaves; ++v) M = fmaxf(M, pm[v][h]);
    float Lsum = 0.f, acc = 0.f;
    if (M > -INFINITY) {
#pragma unroll
      for (int v = 0; v < kAttnWaves; ++v) {
        const float e_v = pm[v][h] > -INFINITY ? __expf(pm[v][h] - M) : 0.f;
        Lsum += e_v * pl[v][h];
        acc += e_v * po[v][h][d];
      }
    }
    part[32 + e] = acc;
    if (d == 0) {
      part[h] = M;
      part[16 + h] = Lsum;
    }
  }
}

// Merge the kAttnSplits partials of every (row, group) by log-sum-exp.
__global__ __launch_bounds__(256) void msa_combine_kernel(MsaParams p) {
  const int tg = blockIdx.x, t = tg / p.hkv, grp = tg - t * p.hkv;
  const float* part = p.part + (int64_t)tg * kAttnSplits * kMsaPartFloats;
  for (int e = threadIdx.x; e < 16 * kD; e += 256) {
    const int h = e / kD, d = e - h * kD;
    if (h >= p.G) continue;
    float M = -INFINITY;
#pragma unroll
    for (int sp = 0; sp < kAttnSplits; ++sp) M = fmaxf(M, part[sp * kMsaPartFloats + h]);
    float Lsum = 0.f, acc = 0.f;
    if (M > -INFINITY) {
#pragma unroll
      for (int sp = 0; sp < kAttnSplits; ++sp) {
        const float* q = part + sp * kMsaPartFloats;
        const float e_s = q[h] > -INFINITY ? __expf(q[h] - M) : 0.f;
        Lsum += e_s * q[16 + h];
        acc += e_s * q[32 + e];
      }
    }
    const int64_t oh = (int64_t)t * p.hq + grp * p.G + h;
    p.out[oh * kD + d] = Lsum > 0.f ? p.v_scale * acc / Lsum : 0.f;
    if (d == 0 && p.lse) p.lse[oh] = Lsum > 0.f ? M + __logf(Lsum) : -INFINITY;
  }
}

}  // namespace

dsa_status launch_msa(const MsaParams& p, int nblk_max, hipStream_t stream) {
  hipLaunchKernelGGL(msa_index_kernel, dim3((nblk_max + kIdxBlocks - 1) / kIdxBlocks, p.R), dim3(256), 0, stream, p);
  hipLaunchKernelGGL(msa_select_kernel, dim3(p.T * p.hkv), dim3(256), 0, stream, p);
  hipLaunchKernelGGL(msa_attn_kernel, dim3(p.T * p.hkv, kAttnSplits), dim3(64 * kAttnWaves), 0, stream, p);
  hipLaunchKernelGGL(msa_combine_kernel, dim3(p.T * p.hkv), dim3(256), 0, stream, p);
  return hipGetLastError() == hipSuccess ? DSA_OK : DSA_ERR_HIP;
}

DSA_DEBUG_TAKE(msa)

}  // namespace dsa
