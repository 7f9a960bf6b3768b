// Front end of a DSA layer step: index-query quantisation and new-token cache
// insertion.
//
// Kimi K3.1 Pro day-0 page, "Low-latency decoding: the fused DSA decode path":
// the indexer front end quantises the index query to FP8 or MXFP4 with the
// head weights folded into the quantisation and writes the new token's index
// key; the MLA query step writes the new token's latent into the KV cache.
// Formats: same page, "One KV cache, three states"; AMD section "native MXFP4
// indexer".  Scale rules:
//   FP8 row   s = amax / 448 (1 for an all-zero row), code = E4M3(x / s)
//   MXFP4     per 32 values E8M0 = (fp32 exponent field of amax) - 2, clamped
//             to 0..254, code = E2M1(x / 2^(E8M0 - 127))
//   NVFP4     per 16 values s = E4M3(amax / 6), code = E2M1(x / value(s)) (0
//             when s decodes to 0); the 64 rope dims of a latent are E4M3(x),
//             unscaled; NVFP4 index keys (MiniMax-M3.1-Flash page, "Quick
//             start") take the same rule over their 128 dims
//   folding   FP8 query rows also give w' = w * s: w' ReLU(code . k) equals
//             w ReLU((s code) . k) because s > 0
// E4M3 / E2M1 codes are the nearest value, ties to the even code, saturating
// at 448 / 6, and a zero result is stored as +0.  Every division that decides
// a code is an IEEE fp32 division (correctly rounded).
//
// quantize_q: one 256-thread workgroup per query row, 8 threads per head (16
// dims each, two 16-byte loads).  cache_insert: one wave per new token; the
// token's page comes from the block table, its slot from its position.
#include "common.h"
#include "kernels.h"

namespace dsa {

// fp32 -> E4M3FN code: round to nearest even on the fp32 bits, saturating.
__device__ __forceinline__ uint32_t e4m3_code(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fminf(fabsf(v), 448.f);
  const uint32_t ab = __float_as_uint(a);
  int e = (int)(ab >> 23) - 127;
  uint32_t code;
  if (e < -6) {
    // below the smallest normal: a multiple of 2^-9 (8 of them = 2^-6)
    code = (uint32_t)__builtin_rintf(a * 512.f);
  } else {
    const uint32_t mant = ab & 0x7FFFFFu;
    uint32_t m3 = mant >> 20;
    const uint32_t rest = mant & 0xFFFFFu;
    if (rest > 0x80000u || (rest == 0x80000u && (m3 & 1u))) ++m3;
    if (m3 == 8u) {
      m3 = 0;
      ++e;
    }
    code = ((uint32_t)(e + 7) << 3) | m3;
  }
  return code == 0 ? 0u : (code | sign);
}

// fp32 -> 4-bit E2M1 code: thresholds at the midpoints, ties to the even code.
__device__ __forceinline__ uint32_t e2m1_code(float v) {
  const float a = fminf(fabsf(v), 6.f);
  const uint32_t c = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                     (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) + (uint32_t)(a > 5.f);
  return c == 0 ? 0u : (c | ((__float_as_uint(v) >> 28) & 0x8u));
}

// E8M0 code of an MX block from its amax (fp32 exponent field - 2, clamped).
__device__ __forceinline__ uint32_t mx_code(float amax) {
  const int f = (int)((__float_as_uint(amax) >> 23) & 0xFFu) - 2;
  return (uint32_t)min(max(f, 0), 254);
}
__device__ __forceinline__ float pow2f(int e) {  // 2^e for e in -127 .. 127, exact
  return e >= -126 ? __uint_as_float((uint32_t)(e + 127) << 23) : __uint_as_float(0x00400000u);
}

__device__ __forceinline__ float amax_lanes(float a, int width) {
  for (int o = 1; o < width; o <<= 1) a = fmaxf(a, __shfl_xor(a, o));
  return a;
}

__device__ __forceinline__ void load_bf16x8(const uint16_t* src, float (&x)[8]) {
  const i32x4 v = *reinterpret_cast<const i32x4*>(src);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = bf16_lo((uint32_t)v[i]);
    x[2 * i + 1] = bf16_hi((uint32_t)v[i]);
  }
}

template <int FMT>
__global__ __launch_bounds__(256) void quantize_q_kernel(QuantQParams p) {
  const int t = blockIdx.x, tid = threadIdx.x;
  const int h = tid >> 3, j = tid & 7;  // head, sixteenth of its 128 dims
  const int64_t row = (int64_t)t * 32 + h;
  float x[16];
  {
    float a[8], b[8];
    load_bf16x8(p.q + row * 128 + 16 * j, a);
    load_bf16x8(p.q + row * 128 + 16 * j + 8, b);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      x[i] = a[i];
      x[8 + i] = b[i];
    }
  }
  float am = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) am = fmaxf(am, fabsf(x[i]));
  if (FMT == DSA_Q_FP8) {
    am = amax_lanes(am, 8);
    const float s = am > 0.f ? am / 448.f : 1.f;
    uint32_t w4[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w4[i] = e4m3_code(x[4 * i] / s) | (e4m3_code(x[4 * i + 1] / s) << 8) | (e4m3_code(x[4 * i + 2] / s) << 16) |
              (e4m3_code(x[4 * i + 3] / s) << 24);
    *reinterpret_cast<i32x4*>(p.out + row * 128 + 16 * j) = i32x4{(int)w4[0], (int)w4[1], (int)w4[2], (int)w4[3]};
    if (j == 0) {
      static_cast<float*>(p.scale)[row] = s;
      if (p.w_folded) p.w_folded[row] = p.w[row] * s;
    }
  } else {
    am = amax_lanes(am, 2);  // a 32-value block is two threads
    const uint32_t e8 = mx_code(am);
    const float s = pow2f((int)e8 - 127);
    uint32_t w2[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      uint32_t v = 0;
#pragma unroll
      for (int u = 0; u < 8; ++u) v |= e2m1_code(x[8 * i + u] / s) << (4 * u);
      w2[i] = v;
    }
    *reinterpret_cast<i32x2*>(p.out + row * 64 + 8 * j) = i32x2{(int)w2[0], (int)w2[1]};
    if ((j & 1) == 0) static_cast<uint8_t*>(p.scale)[row * 4 + (j >> 1)] = (uint8_t)e8;
  }
}

// Physical page of position pos of request r (-1: outside the table or pool).
__device__ __forceinline__ int insert_page(const InsertParams& p, int r, int pos, int plog2, int num_pages) {
  int pg;
  if (p.block_table) {
    const int lp = pos >> plog2;
    DSA_DEBUG_NOTE(lp >= p.bt_stride, DSA_DEBUG_ROW_OUTSIDE);
    if (lp >= p.bt_stride) return -1;
    pg = p.block_table[(int64_t)r * p.bt_stride + lp];
  } else {
    pg = r;
  }
  DSA_DEBUG_NOTE(pg < 0 || pg >= num_pages, DSA_DEBUG_ABSENT_PAGE);
  return (pg >= 0 && pg < num_pages) ? pg : -1;
}

template <int KFMT, int LFMT>
__global__ __launch_bounds__(64) void cache_insert_kernel(InsertParams p) {
  const int i = blockIdx.x, l = threadIdx.x;
  const int r = p.tok_req[i], pos = p.tok_pos[i];
  DSA_DEBUG_NOTE(r < 0 || r >= p.R, DSA_DEBUG_REQ_OUTSIDE);
  if (r < 0 || r >= p.R || pos < 0) return;
  if (KFMT != 0) {
    const int pg = insert_page(p, r, pos, p.key_plog2, p.key_num_pages);
    if (pg >= 0) {
      const int P = 1 << p.key_plog2, slot = pos & (P - 1);
      uint8_t* page = p.keys + (int64_t)pg * p.key_page_bytes;
      const uint32_t w = reinterpret_cast<const uint32_t*>(p.key_vals + (int64_t)i * 128)[l];  // dims 2l, 2l+1
      const float x0 = bf16_lo(w), x1 = bf16_hi(w);
      const float a = fmaxf(fabsf(x0), fabsf(x1));
      if (KFMT == DSA_KEY_FP8) {
        const float am = amax_lanes(a, 64);
        const float s = am > 0.f ? am / 448.f : 1.f;
        reinterpret_cast<uint16_t*>(page + slot * 128)[l] = (uint16_t)(e4m3_code(x0 / s) | (e4m3_code(x1 / s) << 8));
        if (l == 0) *reinterpret_cast<float*>(page + P * 128 + slot * 4) = s;
      } else if (KFMT == DSA_KEY_MXFP4) {
        const float am = amax_lanes(a, 16);  // 32 dims = 16 lanes
        const uint32_t e8 = mx_code(am);
        const float s = pow2f((int)e8 - 127);
        page[slot * 64 + l] = (uint8_t)(e2m1_code(x0 / s) | (e2m1_code(x1 / s) << 4));
        if ((l & 15) == 0) page[P * 64 + slot * 4 + (l >> 4)] = (uint8_t)e8;
      } else {
        const float am = amax_lanes(a, 8);  // 16 dims = 8 lanes
        const uint32_t sc = e4m3_code(am / 6.f);
        const float sv = e4m3_to_f32(sc);
        page[slot * 64 + l] = sv > 0.f ? (uint8_t)(e2m1_code(x0 / sv) | (e2m1_code(x1 / sv) << 4)) : (uint8_t)0;
        if ((l & 7) == 0) page[P * 64 + slot * 8 + (l >> 3)] = (uint8_t)sc;
      }
    }
  }
  if (LFMT != 0) {
    const int pg = insert_page(p, r, pos, p.lat_plog2, p.lat_num_pages);
    if (pg < 0) return;
    const int P = 1 << p.lat_plog2, slot = pos & (P - 1);
    const uint16_t* src = p.lat_vals + (int64_t)i * 576;
    if (LFMT == DSA_LAT_BF16) {
      uint16_t* row = reinterpret_cast<uint16_t*>(p.lat + (int64_t)pg * p.lat_page_bytes + (int64_t)slot * 1152);
#pragma unroll
      for (int jj = 0; jj < 9; ++jj) row[64 * jj + l] = src[64 * jj + l];
    } else if (LFMT == DSA_LAT_FP8) {
      uint8_t* row = p.lat + (int64_t)pg * p.lat_page_bytes + (int64_t)slot * 640;
      float x[9], a = 0.f;
#pragma unroll
      for (int jj = 0; jj < 9; ++jj) {
        x[jj] = __uint_as_float((uint32_t)src[64 * jj + l] << 16);
        a = fmaxf(a, fabsf(x[jj]));
      }
      const float am = amax_lanes(a, 64);
      const float s = am > 0.f ? am / 448.f : 1.f;
#pragma unroll
      for (int jj = 0; jj < 9; ++jj) row[64 * jj + l] = (uint8_t)e4m3_code(x[jj] / s);
      if (l == 0) *reinterpret_cast<float*>(row + 576) = s;
    } else {
      uint8_t* row = p.lat + (int64_t)pg * p.lat_page_bytes + (int64_t)slot * 384;
      float x[8];
      load_bf16x8(src + 8 * l, x);  // dims 8l .. 8l+7 of the 512 value dims
      float a = 0.f;
#pragma unroll
      for (int u = 0; u < 8; ++u) a = fmaxf(a, fabsf(x[u]));
      const float am = amax_lanes(a, 2);  // a 16-dim block is two lanes
      const uint32_t sc = e4m3_code(am / 6.f);
      const float sv = e4m3_to_f32(sc);
      uint32_t v = 0;
      if (sv > 0.f) {
#pragma unroll
        for (int u = 0; u < 8; ++u) v |= e2m1_code(x[u] / sv) << (4 * u);
      }
      *reinterpret_cast<uint32_t*>(row + 4 * l) = v;
      if ((l & 1) == 0) row[256 + (l >> 1)] = (uint8_t)sc;
      row[288 + l] = (uint8_t)e4m3_code(__uint_as_float((uint32_t)src[512 + l] << 16));  // rope dim 512 + l
    }
  }
}

dsa_status launch_quantize_q(const QuantQParams& p, hipStream_t stream) {
  if (p.fmt == DSA_Q_FP8)
    hipLaunchKernelGGL(quantize_q_kernel<DSA_Q_FP8>, dim3(p.T), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(quantize_q_kernel<DSA_Q_MXFP4>, dim3(p.T), dim3(256), 0, stream, p);
  return hipGetLastError() == hipSuccess ? DSA_OK : DSA_ERR_HIP;
}

dsa_status launch_cache_insert(const InsertParams& p, hipStream_t stream) {
  const dim3 grid(p.n), block(64);
  const int k = p.key_vals ? p.key_fmt : 0, lf = p.lat_vals ? p.lat_fmt : 0;
#define DSA_INSERT(K, L) \
  if (k == (K) && lf == (L)) hipLaunchKernelGGL((cache_insert_kernel<K, L>), grid, block, 0, stream, p)
  DSA_INSERT(DSA_KEY_FP8, 0);
  DSA_INSERT(DSA_KEY_MXFP4, 0);
  DSA_INSERT(0, DSA_LAT_BF16);
  DSA_INSERT(0, DSA_LAT_FP8);
  DSA_INSERT(0, DSA_LAT_NVFP4);
  DSA_INSERT(DSA_KEY_FP8, DSA_LAT_BF16);
  DSA_INSERT(DSA_KEY_FP8, DSA_LAT_FP8);
  DSA_INSERT(DSA_KEY_FP8, DSA_LAT_NVFP4);
  DSA_INSERT(DSA_KEY_MXFP4, DSA_LAT_BF16);
  DSA_INSERT(DSA_KEY_MXFP4, DSA_LAT_FP8);
  DSA_INSERT(DSA_KEY_MXFP4, DSA_LAT_NVFP4);
  DSA_INSERT(DSA_KEY_NVFP4, 0);
  DSA_INSERT(DSA_KEY_NVFP4, DSA_LAT_BF16);
  DSA_INSERT(DSA_KEY_NVFP4, DSA_LAT_FP8);
  DSA_INSERT(DSA_KEY_NVFP4, DSA_LAT_NVFP4);
#undef DSA_INSERT
  return hipGetLastError() == hipSuccess ? DSA_OK : DSA_ERR_HIP;
}

DSA_DEBUG_TAKE(quant)

}  // namespace dsa
