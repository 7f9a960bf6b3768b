// Lightning indexer on FP8 MFMA: FP8 queries (codes x per-(row, head) scale)
// against FP8 paged keys -- the compute-bound prefill shape.
//
//   score(t, s) = ks_s * sum_h (w[t,h] * qs[t,h]) * max(0, qcode[t,h,:] . kcode_s)
//
// The per-row query scale and the per-token key scale are positive, so they
// pull out of the ReLU and the dot product runs on raw E4M3 codes with
// v_mfma_scale_f32_16x16x128_f8f6f4 (unit block scales), one instruction per
// 16 heads x 16 keys (the 128-dim dot is a single K step).  Kimi K3.1 Pro
// day-0 page, "Prefill: shard attention by token": the indexer's cost is
// quadratic in the context; MiniMax-M3.1 day-0 page, AMD "NVFP4 indexer DCP":
// the 16x16x128 FP8 MFMA needs 16 rows of queries to fill.
//
// Work split: a workgroup owns 16 query rows of one request (4 per wave, held
// in registers as A fragments: 2 head halves x 32 bytes per lane) and sweeps a
// segment of the keys in tiles of 128 staged in LDS (rows padded to 144 bytes
// so the 16 key rows a fragment read touches fall in distinct banks).  The
// epilogue is the decode indexer's: ReLU-weighted head sum in-lane, then a
// reduce-scatter over the four lane groups, one score per lane, 64 coalesced
// scores per (row, 64 keys).  Keys at or past a row's visible count are not
// written (causal prefill).
#include "common.h"
#include "kernels.h"

namespace dsa {

constexpr int kF8BM = 16;    // query rows per workgroup
constexpr int kF8BN = 128;   // keys per LDS tile
constexpr int kF8KPad = 144; // bytes per key row in LDS

__global__ __launch_bounds__(256) void indexer_fp8_kernel(IndexerParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t kl[kF8BN * kF8KPad];
  __shared__ float kscale[kF8BN];
  __shared__ float wl[kF8BM * 32];  // w * q_scale per row and head
  __shared__ int s_vmax[4];
  __shared__ int pg_lds[16384 / 16 + 1];  // page ids of this workgroup's key segment

  const int r = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int rs = p.req_row_start[r], re = p.req_row_start[r + 1];
  const int row0 = rs + blockIdx.y * kF8BM;
  if (row0 >= re) return;
  const int nrows = min(kF8BM, re - row0);
  const int P = 1 << p.plog2;

  // visible range of this workgroup's rows
  int vm = 0;
  if (tid < nrows) vm = clamp_vis(p.tok_vis[row0 + tid], p.max_vis);
  for (int o = 32; o > 0; o >>= 1) vm = max(vm, __shfl_xor(vm, o));
  if (lane == 0) s_vmax[wave] = vm;
  for (int i = tid; i < kF8BM * 32; i += 256) {
    const int j = i >> 5;
    wl[i] = j < nrows ? p.w[(int64_t)(row0 + j) * 32 + (i & 31)] * p.q_scale[(int64_t)(row0 + j) * 32 + (i & 31)]
                      : 0.f;
  }
  __syncthreads();
  const int vmax = max(max(s_vmax[0], s_vmax[1]), max(s_vmax[2], s_vmax[3]));
  const int kb = blockIdx.x * p.chunk;
  if (kb >= vmax) return;
  const int ke = min(kb + p.chunk, vmax);
  const int lp0 = kb >> p.plog2;
  const int last = ((ke - 1) >> p.plog2) - lp0;  // last staged page entry
  for (int i = tid; i <= last; i += 256) pg_lds[i] = phys_page(p.block_table, p.bt_stride, r, lp0 + i, p.num_pages);
  __syncthreads();

  // A fragments: rows 4*wave + j, head halves hh, lane (g, c): head 16hh + c,
  // dims 32g .. 32g+31 (32 E4M3 bytes)
  i32x8 qa[4][2];
  int vis[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int jr = 4 * wave + j;
    vis[j] = 0;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      i32x4 lo = {0, 0, 0, 0}, hi = lo;
      if (jr < nrows) {
        const uint8_t* qp = p.q8 + ((int64_t)(row0 + jr) * 32 + 16 * hh + c) * 128 + 32 * g;
        lo = ld16(qp);
        hi = ld16(qp + 16);
      }
      qa[j][hh] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
    if (jr < nrows) vis[j] = clamp_vis(p.tok_vis[row0 + jr], p.max_vis);
  }
  f32x4 wv[4][2];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    wv[j][0] = *reinterpret_cast<const f32x4*>(&wl[(4 * wave + j) * 32 + 4 * g]);
    wv[j][1] = *reinterpret_cast<const f32x4*>(&wl[(4 * wave + j) * 32 + 16 + 4 * g]);
  }

  // key tile loader: 128 keys x 128 B = 1024 chunks of 16 B, 4 per thread.
  // Every read is issued unconditionally (a read under a branch waited for the
  // one before): a key past the segment or on an absent page reads the
  // clamped / page-0 address; its scale becomes -inf on an absent page (the
  // score is replaced by -inf) and a key past the segment is never stored.
  i32x4 kraw[4];
  float sraw = 0.f;  // scale of key k0 + (tid & 127) as read
  bool sok = false;  // ... on a present page (else the key's scale is -inf)
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ch = tid + 256 * i;
      const int key = ch >> 3, part = ch & 7;
      const int s = k0 + key;
      const int pg = pg_lds[min((s >> p.plog2) - lp0, last)];
      kraw[i] = ld16(p.keys + (int64_t)max(pg, 0) * p.page_bytes + (s & (P - 1)) * 128 + part * 16);
    }
    {
      // every thread reads a scale (threads 128 .. 255 repeat 0 .. 127); the
      // absent-page select waits until the scale is staged, so nothing here
      // waits for the read
      const int s = k0 + (tid & (kF8BN - 1));
      const int pg = pg_lds[min((s >> p.plog2) - lp0, last)];
      sraw = *reinterpret_cast<const float*>(p.keys + (int64_t)max(pg, 0) * p.page_bytes + P * 128 + (s & (P - 1)) * 4);
      sok = pg >= 0;
    }
  };

  load_tile(kb);
  for (int k0 = kb; k0 < ke; k0 += kF8BN) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ch = tid + 256 * i;
      *reinterpret_cast<i32x4*>(&kl[(ch >> 3) * kF8KPad + (ch & 7) * 16]) = kraw[i];
    }
    if (tid < kF8BN) kscale[tid] = sok ? sraw : -__builtin_inff();
    __syncthreads();

    // issued after the last tile too (reads stay in the staged pages; never
    // used): no branch around the reads
    load_tile(k0 + kF8BN);

#pragma unroll
    for (int q4 = 0; q4 < kF8BN / 64; ++q4) {
      // B fragments of 4 tiles of 16 keys: key c, dims 32g .. 32g+31
      i32x8 kb8[4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const uint8_t* src = &kl[(q4 * 64 + kt * 16 + c) * kF8KPad + 32 * g];
        const i32x4 lo = *reinterpret_cast<const i32x4*>(src);
        const i32x4 hi = *reinterpret_cast<const i32x4*>(src + 16);
        kb8[kt] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
      const int kloc = q4 * 64 + lane;           // key this lane stores
      const float ksv = kscale[kloc];
      const int s = k0 + kloc;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f32x4 acc[4][2];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          acc[kt][0] = mfma16x16x128_fp8(qa[j][0], kb8[kt], f32x4{0.f, 0.f, 0.f, 0.f});
          acc[kt][1] = mfma16x16x128_fp8(qa[j][1], kb8[kt], f32x4{0.f, 0.f, 0.f, 0.f});
        }
        float v[4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          float x = 0.f;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            x += wv[j][0][i] * relu(acc[kt][0][i]);
            x += wv[j][1][i] * relu(acc[kt][1][i]);
          }
          v[kt] = x;
        }
        const float tot = rows_reduce_scatter4(v);
        if (s < vis[j] && s < ke)
          p.scores[(int64_t)(row0 + 4 * wave + j) * p.ld + s] = (ksv == -__builtin_inff()) ? ksv : tot * ksv;
      }
    }
  }
}

dsa_status launch_indexer_fp8(const IndexerParams& p, hipStream_t stream) {
  dim3 grid((p.max_vis + p.chunk - 1) / p.chunk, (p.max_rows_per_req + kF8BM - 1) / kF8BM, p.R);
  hipLaunchKernelGGL(indexer_fp8_kernel, grid, dim3(256), 0, stream, p);
  return hipGetLastError() == hipSuccess ? DSA_OK : DSA_ERR_HIP;
}

DSA_DEBUG_TAKE(indexer_fp8)

}  // namespace dsa
