// Sparse MLA over selected latent rows, and the log-sum-exp merge of splits.
//
//   l_s = sm_scale * q_h . c_s  (576-d latents),  o_h = sum_s softmax(l)_s c_s[0:512]
//
// (Kimi K3.1 Pro day-0 page, "Sparse attention in K3.1 Pro": exact MLA over
// the 2,048 selected tokens; MI355X Kimi K3 page, section 4 "MLA": query heads
// padded 12 -> 16 so the matrix tile fills, history split into pieces that
// are merged afterwards; Kimi K3.1 Pro day-0 page, "Long context: decode
// context parallel": partial outputs merged by log-sum-exp.)
//
// One workgroup = one query row x one split of its selection list x up to
// four 16-head tiles, one wave each (heads padded to a multiple of 16
// in-kernel; padded heads get zero queries and are never written).  With one
// wave per SIMD a wave may hold its 128 accumulator registers, the 72
// registers of its query fragments and the tile temporaries without spills.  For every 32 selected rows:
//   gather   all waves load the rows with 16-byte loads, dequantise them
//            exactly to bf16 (FP8 codes; NVFP4 codes x E4M3 block scale; BF16
//            copied) and store a [32 x 576] tile in LDS.  A per-row FP8 scale
//            is kept aside and folded into the logits and softmax weights.
//   QK       S^T[rows x heads] = Lat . Q^T on v_mfma_f32_16x16x32_bf16: lane
//            (g, c) supplies latent row c and head c over the same dims
//            (k-step kk < 16: nope dims 128g + 8kk..; kk = 16, 17: rope dims
//            512 + 16g + 8(kk-16)..).  The result lands with lane (g, c)
//            holding rows 4g+i of head c -- exactly the A operand the value
//            product needs, so the softmax weights never leave registers.
//   softmax  online, base 2, per head; the head max/sum reduce over the four
//            lane groups with two xor shuffles.
//   PV       O[heads x 512] += P[heads x 32 rows] . V[32 rows x 512]: the V
//            operand needs 8 rows of one column per lane, read as 4x4 bf16
//            blocks (ds_read_b64) and transposed with v_perm_b32.  Lane (g, c)
//            accumulates heads 4g+i at dims 64a + 4c + u.
#include "common.h"
#include "kernels.h"

namespace dsa {

constexpr int kRT = 32;      // selected rows per tile
constexpr int kLPad = 584;   // bf16 per LDS latent row (1168 B: conflict-free row reads)

__device__ __forceinline__ int dim_of(int kk, int g) {
  return kk < 16 ? 128 * g + 8 * kk : 512 + 16 * g + 8 * (kk - 16);
}

template <int FMT>
__device__ __forceinline__ void gather_tile(const MlaParams& p, int t, int j0, int j_end, __bf16* lat,
                                            float* rsc, int* rid) {
  const int tid = threadIdx.x, nth = blockDim.x;
  const int P = 1 << p.plog2;
  if (tid < kRT) {
    const int j = j0 + tid;
    int id = (j < j_end) ? p.rows[(int64_t)t * p.k + j] : -1;
    if (id >= 0 && (id >> p.plog2) >= p.num_pages) id = -1;
    rid[tid] = id;
    float sc = id >= 0 ? 1.f : 0.f;
    if (FMT == DSA_LAT_FP8 && id >= 0) {
      const uint8_t* page = p.lat + (int64_t)(id >> p.plog2) * p.page_bytes;
      sc = *reinterpret_cast<const float*>(page + P * 576 + (id & (P - 1)) * 4);
    }
    rsc[tid] = sc;
  }
  __syncthreads();
  if (FMT == DSA_LAT_FP8) {
    for (int i = tid; i < kRT * 36; i += nth) {
      const int row = i / 36, part = i - row * 36;
      const int id = rid[row];
      i32x4 lo = {0, 0, 0, 0}, hi = {0, 0, 0, 0};
      if (id >= 0) {
        const uint8_t* src = p.lat + (int64_t)(id >> p.plog2) * p.page_bytes + (id & (P - 1)) * 576 + part * 16;
        const i32x4 v = ld16(src);
        const i32x2 a = e4m3x4_to_bf16(v[0]), b = e4m3x4_to_bf16(v[1]);
        const i32x2 c2 = e4m3x4_to_bf16(v[2]), d = e4m3x4_to_bf16(v[3]);
        lo = i32x4{a[0], a[1], b[0], b[1]};
        hi = i32x4{c2[0], c2[1], d[0], d[1]};
      }
      i32x4* dst = reinterpret_cast<i32x4*>(&lat[row * kLPad + part * 16]);
      dst[0] = lo;
      dst[1] = hi;
    }
  } else if (FMT == DSA_LAT_BF16) {
    for (int i = tid; i < kRT * 72; i += nth) {
      const int row = i / 72, part = i - row * 72;
      const int id = rid[row];
      i32x4 v = {0, 0, 0, 0};
      if (id >= 0)
        v = ld16(p.lat + (int64_t)(id >> p.plog2) * p.page_bytes + (int64_t)(id & (P - 1)) * 1152 + part * 16);
      *reinterpret_cast<i32x4*>(&lat[row * kLPad + part * 8]) = v;
    }
  } else {  // NVFP4: 16 code chunks (32 dims each) + 4 rope chunks (16 dims each) per row
    for (int i = tid; i < kRT * 20; i += nth) {
      const int row = i / 20, part = i - row * 20;
      const int id = rid[row];
      i32x4* dst;
      if (part < 16) {
        dst = reinterpret_cast<i32x4*>(&lat[row * kLPad + part * 32]);
        i32x4 o0 = {0, 0, 0, 0}, o1 = o0, o2 = o0, o3 = o0;
        if (id >= 0) {
          const uint8_t* page = p.lat + (int64_t)(id >> p.plog2) * p.page_bytes;
          const int slot = id & (P - 1);
          const i32x4 v = ld16(page + slot * 256 + part * 16);
          const uint32_t s2 = *reinterpret_cast<const uint16_t*>(page + 256 * P + slot * 32 + part * 2);
          const float sa = e4m3_to_f32(s2 & 0xFFu), sb = e4m3_to_f32(s2 >> 8);
          o0 = __builtin_bit_cast(i32x4, e2m1x8_times(v[0], sa));
          o1 = __builtin_bit_cast(i32x4, e2m1x8_times(v[1], sa));
          o2 = __builtin_bit_cast(i32x4, e2m1x8_times(v[2], sb));
          o3 = __builtin_bit_cast(i32x4, e2m1x8_times(v[3], sb));
        }
        dst[0] = o0;
        dst[1] = o1;
        dst[2] = o2;
        dst[3] = o3;
      } else {
        const int q4 = part - 16;
        dst = reinterpret_cast<i32x4*>(&lat[row * kLPad + 512 + q4 * 16]);
        i32x4 lo = {0, 0, 0, 0}, hi = lo;
        if (id >= 0) {
          const uint8_t* page = p.lat + (int64_t)(id >> p.plog2) * p.page_bytes;
          const i32x4 v = ld16(page + 288 * P + (id & (P - 1)) * 64 + q4 * 16);
          const i32x2 a = e4m3x4_to_bf16(v[0]), b = e4m3x4_to_bf16(v[1]);
          const i32x2 c2 = e4m3x4_to_bf16(v[2]), d = e4m3x4_to_bf16(v[3]);
          lo = i32x4{a[0], a[1], b[0], b[1]};
          hi = i32x4{c2[0], c2[1], d[0], d[1]};
        }
        dst[0] = lo;
        dst[1] = hi;
      }
    }
  }
}

template <int FMT>
__global__ __launch_bounds__(256) void mla_kernel(MlaParams p) {
  __shared__ __attribute__((aligned(16))) __bf16 lat[kRT * kLPad];
  __shared__ float rsc[kRT];
  __shared__ int rid[kRT];

  const int split = blockIdx.x, t = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, ht = blockIdx.z * 4 + (tid >> 6);
  const int g = lane >> 4, c = lane & 15;
  const int j_begin = split * p.split_len;
  const int j_end = min(j_begin + p.split_len, p.k);

  // queries of head 16*ht + c as B fragments (zero for padded heads)
  const int head = 16 * ht + c;
  bf16x8 qf[18];
  if (head < p.H) {
    const __bf16* qp = p.q + ((int64_t)t * p.H + head) * 576;
#pragma unroll
    for (int kk = 0; kk < 18; ++kk) qf[kk] = __builtin_bit_cast(bf16x8, ld16(qp + dim_of(kk, g)));
  } else {
#pragma unroll
    for (int kk = 0; kk < 18; ++kk) qf[kk] = bf16x8{};
  }

  f32x4 O[32];
#pragma unroll
  for (int x = 0; x < 32; ++x) O[x] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -__builtin_inff(), l = 0.f;  // running max (log2 units) and sum, head c

  for (int j0 = j_begin; j0 < j_end; j0 += kRT) {
    __syncthreads();
    gather_tile<FMT>(p, t, j0, j_end, lat, rsc, rid);
    __syncthreads();

    // ---- QK: S^T tile, rows 16*nt + 4g + i of head c
    f32x4 s[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      s[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
      const __bf16* lrow = &lat[(16 * nt + c) * kLPad];
#pragma unroll
      for (int kk = 0; kk < 18; ++kk) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(lrow + dim_of(kk, g));
        s[nt] = mfma16x16x32(a, qf[kk], s[nt]);
      }
    }
    // ---- online softmax for head c
    float lg[8], rs[8];
    float tmax = -__builtin_inff();
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * nt + 4 * g + i;
        const float sc = rsc[row];
        rs[nt * 4 + i] = sc;
        const float v = rid[row] >= 0 ? s[nt][i] * p.sm_log2 * sc : -__builtin_inff();
        lg[nt * 4 + i] = v;
        tmax = fmaxf(tmax, v);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float mnew = fmaxf(m, tmax);
    const float alpha = (mnew == -__builtin_inff()) ? 1.f : exp2f(m - mnew);
    float psum = 0.f;
    float pw[8];
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      const float e = (lg[x] == -__builtin_inff()) ? 0.f : exp2f(lg[x] - mnew);
      psum += e;
      pw[x] = e * rs[x];  // FP8 row scale enters the value product here
    }
    psum = wave_sum_xor_16_32(psum);
    l = l * alpha + psum;
    m = mnew;
    const i32x4 pa4 = {(int)pack_bf16x2(pw[0], pw[1]), (int)pack_bf16x2(pw[2], pw[3]),
                       (int)pack_bf16x2(pw[4], pw[5]), (int)pack_bf16x2(pw[6], pw[7])};
    const bf16x8 pa = __builtin_bit_cast(bf16x8, pa4);

    // ---- rescale accumulators (heads 4g+i) when any running max moved
    if (__ballot(alpha != 1.f)) {
      float ai[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) ai[i] = __shfl(alpha, 4 * g + i);
#pragma unroll
      for (int x = 0; x < 32; ++x)
#pragma unroll
        for (int i = 0; i < 4; ++i) O[x][i] *= ai[i];
    }

    // ---- PV
    int rr[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) rr[j] = (j < 4) ? (4 * g + j) : (16 + 4 * g + j - 4);
#pragma unroll
    for (int a = 0; a < 8; ++a) {
      i32x2 rv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) rv[j] = *reinterpret_cast<const i32x2*>(&lat[rr[j] * kLPad + 64 * a + 4 * c]);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int half = u >> 1;
        const uint32_t sel = (u & 1) ? 0x07060302u : 0x05040100u;
        i32x4 f;
#pragma unroll
        for (int d = 0; d < 4; ++d)
          f[d] = (int)__builtin_amdgcn_perm((uint32_t)rv[2 * d + 1][half], (uint32_t)rv[2 * d][half], sel);
        O[a * 4 + u] = mfma16x16x32(pa, __builtin_bit_cast(bf16x8, f), O[a * 4 + u]);
      }
    }
  }

  // ---- epilogue: normalise heads 4g+i
  float li[4], mi[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    li[i] = __shfl(l, 4 * g + i);
    mi[i] = __shfl(m, 4 * g + i);
  }
  const bool final_out = p.nsplit == 1;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = 16 * ht + 4 * g + i;
    if (h >= p.H) continue;
    const float inv = li[i] > 0.f ? 1.f / li[i] : 0.f;
    float* dst = final_out ? p.out + ((int64_t)t * p.H + h) * 512
                           : p.part_o + (((int64_t)t * p.nsplit + split) * p.H + h) * 512;
#pragma unroll
    for (int a = 0; a < 8; ++a) {
      f32x4 v = {O[a * 4 + 0][i] * inv, O[a * 4 + 1][i] * inv, O[a * 4 + 2][i] * inv, O[a * 4 + 3][i] * inv};
      *reinterpret_cast<f32x4*>(dst + 64 * a + 4 * c) = v;
    }
    if (c == 0) {
      const float lse = li[i] > 0.f ? (mi[i] + __log2f(li[i])) * 0.69314718055994531f : -__builtin_inff();
      if (final_out) {
        if (p.lse) p.lse[(int64_t)t * p.H + h] = lse;
      } else {
        p.part_lse[((int64_t)t * p.nsplit + split) * p.H + h] = lse;
      }
    }
  }
}

__global__ __launch_bounds__(128) void mla_combine_kernel(MlaParams p) {
  const int h = blockIdx.x, t = blockIdx.y;
  const int tid = threadIdx.x;
  const float* pl = p.part_lse + (int64_t)t * p.nsplit * p.H + h;
  float mx = -__builtin_inff();
  for (int s = 0; s < p.nsplit; ++s) mx = fmaxf(mx, pl[(int64_t)s * p.H]);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  if (mx != -__builtin_inff()) {
    for (int s = 0; s < p.nsplit; ++s) {
      const float ls = pl[(int64_t)s * p.H];
      if (ls == -__builtin_inff()) continue;
      const float w = __expf(ls - mx);
      wsum += w;
      const f32x4 v =
          *reinterpret_cast<const f32x4*>(p.part_o + (((int64_t)t * p.nsplit + s) * p.H + h) * 512 + 4 * tid);
      acc += w * v;
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  *reinterpret_cast<f32x4*>(p.out + ((int64_t)t * p.H + h) * 512 + 4 * tid) = acc * inv;
  if (tid == 0 && p.lse) p.lse[(int64_t)t * p.H + h] = wsum > 0.f ? mx + __logf(wsum) : -__builtin_inff();
}

dsa_status launch_mla(const MlaParams& p, hipStream_t stream) {
  // at most four head tiles (one wave each) per workgroup; more go to grid.z
  dim3 grid(p.nsplit, p.T, (p.ntiles + 3) / 4), block(64 * (p.ntiles < 4 ? p.ntiles : 4));
  switch (p.fmt) {
    case DSA_LAT_BF16: hipLaunchKernelGGL(mla_kernel<DSA_LAT_BF16>, grid, block, 0, stream, p); break;
    case DSA_LAT_FP8: hipLaunchKernelGGL(mla_kernel<DSA_LAT_FP8>, grid, block, 0, stream, p); break;
    default: hipLaunchKernelGGL(mla_kernel<DSA_LAT_NVFP4>, grid, block, 0, stream, p); break;
  }
  if (p.nsplit > 1) hipLaunchKernelGGL(mla_combine_kernel, dim3(p.H, p.T), dim3(128), 0, stream, p);
  return hipGetLastError() == hipSuccess ? DSA_OK : DSA_ERR_HIP;
}

}  // namespace dsa
