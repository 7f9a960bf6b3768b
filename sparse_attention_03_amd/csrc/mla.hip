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
// registers of its query fragments and the tile temporaries without spills.
// For every 16 selected rows:
//   gather   all waves load the rows with 16-byte loads (four lanes per row,
//            64 contiguous bytes per load instruction per row), dequantise
//            them exactly to bf16 (FP8 codes; NVFP4 codes x E4M3 block scale;
//            BF16 copied) and store a [16 x 576] tile in LDS.  A per-row FP8 scale
//            is kept aside and folded into the logits and softmax weights.
//            Software pipeline: the loads of tile i+1 are issued into
//            registers before tile i computes, and the row ids of tile i+2
//            are fetched a step earlier still, so HBM latency overlaps the
//            MFMA work instead of stalling every tile.
//   QK       S^T[rows x heads] = Lat . Q^T on v_mfma_f32_16x16x32_bf16: lane
//            (g, c) supplies latent row c and head c over the same dims
//            (k-step kk < 16: nope dims 128g + 8kk..; kk = 16, 17: rope dims
//            512 + 16g + 8(kk-16)..).  The result lands with lane (g, c)
//            holding rows 4g+i of head c -- exactly the A operand the value
//            product needs, so the softmax weights never leave registers.
//   softmax  online, base 2, per head; the head max/sum reduce over the four
//            lane groups with two xor shuffles.  The running max only moves
//            when a tile exceeds it by 2^8, so the 128 accumulators are
//            rescaled rarely instead of on almost every tile.
//   PV       O[heads x 512] += P[heads x 16 rows] . V[16 rows x 512] on
//            v_mfma_f32_16x16x16_bf16: the V operand needs 4 rows of one
//            column per lane, which one transposing LDS read
//            (ds_read_b64_tr_b16) delivers per MFMA.  Lane (g, c)
//            accumulates heads 4g+i at dims 64a + 16u + c.
#include <mutex>

#include "common.h"
#include "kernels.h"

namespace dsa {

constexpr int kRT = 16;      // selected rows per tile
constexpr int kLPad = 584;   // bf16 per LDS latent row (1168 B: conflict-free row reads)

__device__ __forceinline__ int dim_of(int kk, int g) {
  return kk < 16 ? 128 * g + 8 * kk : 512 + 16 * g + 8 * (kk - 16);
}

constexpr float kRescaleLog2 = 8.f;  // running max moves only when it grows by 2^8

// Gather geometry: a row is cut into 64-byte segments; lane l of every wave
// owns row (l >> 2) of the 16-row tile and chunk (l & 3) of each segment, and
// wave w takes segments w, w + NW, ...  The row address is therefore computed
// once per tile and every chunk is an immediate offset from it.
template <int FMT> struct Geo;
template <> struct Geo<DSA_LAT_FP8> { static constexpr int SEGS = 9; };    // 576 E4M3
template <> struct Geo<DSA_LAT_BF16> { static constexpr int SEGS = 18; };  // 576 bf16
template <> struct Geo<DSA_LAT_NVFP4> { static constexpr int SEGS = 5; };  // 4 x 128 E2M1, 64 rope

// Row layout inside a latent page: every row padded to whole 128-byte lines
// with all of its bytes inside, so a gathered row costs only its own lines.
template <int FMT> struct LatRow {
  static constexpr int kBytes = FMT == DSA_LAT_BF16 ? 1152 : FMT == DSA_LAT_FP8 ? 640 : 384;
  static constexpr int kScale = 576;   // FP8 row: [576 E4M3][fp32 scale][pad]
  static constexpr int kScales = 256;  // NVFP4 row: [256 B E2M1][32 E4M3 block scales]
  static constexpr int kRope = 288;    //            [64 E4M3 rope][pad]
};

struct RowPtr {
  const uint8_t* data;   // FP8/BF16 row, NVFP4 codes
  const uint8_t* aux;    // NVFP4 block scales
  const uint8_t* rope;   // NVFP4 rope
};

__device__ __forceinline__ bool row_ok(int id, const MlaParams& p) {
  DSA_DEBUG_NOTE((id >> p.plog2) >= p.num_pages, DSA_DEBUG_ROW_OUTSIDE);
  return id >= 0 && (id >> p.plog2) < p.num_pages;
}

template <int FMT>
__device__ __forceinline__ RowPtr row_ptr(const MlaParams& p, int id, int P) {
  RowPtr r{nullptr, nullptr, nullptr};
  if (!row_ok(id, p)) return r;
  const uint8_t* row = p.lat + (int64_t)(id >> p.plog2) * p.page_bytes + (int64_t)(id & (P - 1)) * LatRow<FMT>::kBytes;
  r.data = row;
  if (FMT == DSA_LAT_NVFP4) {
    r.aux = row + LatRow<FMT>::kScales;
    r.rope = row + LatRow<FMT>::kRope;
  }
  return r;
}

// Load segments sp = s0, s0 + NW, ... (SPT of them) of this lane's row.
template <int FMT, int NW, int SPT>
__device__ __forceinline__ void seg_load(const RowPtr& rp, int s0, int q, i32x4 (&raw)[SPT], uint32_t (&aux)[SPT]) {
  constexpr int SEGS = Geo<FMT>::SEGS;
#pragma unroll
  for (int i = 0; i < SPT; ++i) {
    const int sp = s0 + i * NW;
    raw[i] = i32x4{0, 0, 0, 0};
    aux[i] = 0;
    if (sp < SEGS && rp.data) {
      if (FMT == DSA_LAT_NVFP4) {
        if (sp < 4) {
          raw[i] = ld16(rp.data + sp * 64 + q * 16);
          aux[i] = *reinterpret_cast<const uint16_t*>(rp.aux + (sp * 4 + q) * 2);
        } else {
          raw[i] = ld16(rp.rope + q * 16);
        }
      } else {
        raw[i] = ld16(rp.data + sp * 64 + q * 16);
      }
    }
  }
}

// Dequantise the loaded segments into this lane's LDS row.
template <int FMT, int NW, int SPT>
__device__ __forceinline__ void seg_store(__bf16* lrow, int s0, int q, const i32x4 (&raw)[SPT],
                                          const uint32_t (&aux)[SPT]) {
  constexpr int SEGS = Geo<FMT>::SEGS;
#pragma unroll
  for (int i = 0; i < SPT; ++i) {
    const int sp = s0 + i * NW;
    if (sp >= SEGS) continue;
    const i32x4 v = raw[i];
    if (FMT == DSA_LAT_BF16) {
      *reinterpret_cast<i32x4*>(lrow + (sp * 4 + q) * 8) = v;
    } else if (FMT == DSA_LAT_FP8 || sp == 4) {
      const i32x2 a = e4m3x4_to_bf16(v[0]), b = e4m3x4_to_bf16(v[1]);
      const i32x2 c2 = e4m3x4_to_bf16(v[2]), d = e4m3x4_to_bf16(v[3]);
      i32x4* dst = reinterpret_cast<i32x4*>(lrow + (FMT == DSA_LAT_FP8 ? (sp * 4 + q) * 16 : 512 + q * 16));
      dst[0] = i32x4{a[0], a[1], b[0], b[1]};
      dst[1] = i32x4{c2[0], c2[1], d[0], d[1]};
    } else {  // NVFP4 codes: 32 dims, two E4M3 block scales
      const float sa = e4m3_to_f32(aux[i] & 0xFFu), sb = e4m3_to_f32((aux[i] >> 8) & 0xFFu);
      i32x4* dst = reinterpret_cast<i32x4*>(lrow + (sp * 4 + q) * 32);
      dst[0] = __builtin_bit_cast(i32x4, e2m1x8_times(v[0], sa));
      dst[1] = __builtin_bit_cast(i32x4, e2m1x8_times(v[1], sa));
      dst[2] = __builtin_bit_cast(i32x4, e2m1x8_times(v[2], sb));
      dst[3] = __builtin_bit_cast(i32x4, e2m1x8_times(v[3], sb));
    }
  }
}

// One 16-row tile for one 16-head tile: QK from the LDS tile, online softmax
// (lazy rescale), PV into the accumulators of value dims 64*a0 .. 64*(a0+NA)
// (NA = 8: all 512 dims; NA = 4: the half this wave owns).  rv/rsc: row ids
// (-1 = absent) and per-row value multipliers of the tile.
template <int NA>
__device__ __forceinline__ void mla_tile(const MlaParams& p, const __bf16* lat, const float* rsc, const int* rv,
                                         const bf16x8 (&qf)[18], f32x4 (&O)[NA * 4], float& m, float& l, int g, int c,
                                         int a0) {
  // ---- QK: S^T tile, rows 4g + i of head c.  All 18 fragments are read
  // before the first multiply, and the k-steps alternate between two
  // accumulators (two independent chains of nine).
  f32x4 s;
  {
    const __bf16* lrow = &lat[c * kLPad];
    bf16x8 af[18];
#pragma unroll
    for (int kk = 0; kk < 18; ++kk) af[kk] = *reinterpret_cast<const bf16x8*>(lrow + dim_of(kk, g));
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 18; kk += 2) {
      s0 = mfma16x16x32(af[kk], qf[kk], s0);
      s1 = mfma16x16x32(af[kk + 1], qf[kk + 1], s1);
    }
    s = s0 + s1;
  }
  // ---- online softmax for head c
  float lg[4], rs[4];
  float tmax = -__builtin_inff();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 4 * g + i;
    const float sc = rsc[row];
    rs[i] = sc;
    const float v = rv[row] >= 0 ? s[i] * p.sm_log2 * sc : -__builtin_inff();
    lg[i] = v;
    tmax = fmaxf(tmax, v);
  }
  tmax = fmaxf(tmax, xor16(tmax, g));
  tmax = fmaxf(tmax, xor32(tmax, g));
  // lazy rescaling: keep a stale max while the tile stays within 2^8 of it
  // (weights stay <= 256); both O and l use the same max, so the final
  // normalisation is exact
  const float mnew = (m == -__builtin_inff() || tmax > m + kRescaleLog2) ? tmax : m;
  const float alpha = (m == -__builtin_inff()) ? 1.f : exp2_hw(m - mnew);
  // (a max still -inf means every logit so far is -inf: 2^(-inf - 0) = 0)
  const float mref = mnew == -__builtin_inff() ? 0.f : mnew;
  float psum = 0.f;
  float pw[4];
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    const float e = exp2_hw(lg[x] - mref);
    psum += e;
    pw[x] = e * rs[x];  // FP8 row scale enters the value product here
  }
  psum += xor16(psum, g);
  psum += xor32(psum, g);
  l = l * alpha + psum;
  m = mnew;
  const i32x2 pa2 = {(int)pack_bf16x2(pw[0], pw[1]), (int)pack_bf16x2(pw[2], pw[3])};
  const bf16x4 pa = __builtin_bit_cast(bf16x4, pa2);

  // ---- rescale accumulators (heads 4g+i) when any running max moved
  if (__ballot(alpha != 1.f)) {
    float ai[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) ai[i] = __shfl(alpha, 4 * g + i);
#pragma unroll
    for (int x = 0; x < NA * 4; ++x)
#pragma unroll
      for (int i = 0; i < 4; ++i) O[x][i] *= ai[i];
  }

  // ---- PV: O[heads 4g+i][dims 64a + 16u + c] += P . V over the 16 rows.
  // The V operand (rows 4g..4g+3 of one dim per lane) comes from one
  // transposing LDS read per MFMA: lane s of lane group g points at dims
  // d0 + 4(s%4) .. +3 of row 4g + s/4, and ds_read_b64_tr_b16 hands lane c
  // element c%4 of the 8 bytes of lanes 4k + c/4 (k < 4) -- dim d0 + c of
  // rows 4g .. 4g+3.
  const __bf16* vsrc = lat + (4 * g + (c >> 2)) * kLPad + 4 * (c & 3);
#pragma unroll
  for (int aa = 0; aa < NA; ++aa) {
    const int a = a0 + aa;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      typedef short s16x4 __attribute__((ext_vector_type(4)));
      const auto* src = (const __attribute__((address_space(3))) s16x4*)(const void*)(vsrc + 64 * a + 16 * u);
      const s16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16(const_cast<__attribute__((address_space(3))) s16x4*>(src));
      O[aa * 4 + u] = mfma16x16x16(pa, __builtin_bit_cast(bf16x4, vb), O[aa * 4 + u]);
    }
  }
}

// Normalise the accumulators of heads 4g+i (value dims 64*a0 .. 64*(a0+NA))
// and write the output row (one split) or the split's partial output; the
// wave holding dims from 0 writes the LSE.
template <int NA>
__device__ __forceinline__ void mla_finish(const MlaParams& p, const f32x4 (&O)[NA * 4], float m, float l, int t,
                                           int split, int ht, int g, int c, int a0) {
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
    for (int aa = 0; aa < NA; ++aa)
#pragma unroll
      for (int u = 0; u < 4; ++u) dst[64 * (a0 + aa) + 16 * u + c] = O[aa * 4 + u][i] * inv;
    if (c == 0 && a0 == 0) {
      const float lse = li[i] > 0.f ? (mi[i] + __log2f(li[i])) * 0.69314718055994531f : -__builtin_inff();
      if (final_out) {
        if (p.lse) p.lse[(int64_t)t * p.H + h] = lse;
      } else {
        p.part_lse[((int64_t)t * p.nsplit + split) * p.H + h] = lse;
      }
    }
  }
}

template <int FMT, int NW>
__global__ __launch_bounds__(64 * NW) void mla_kernel(MlaParams p) {
  constexpr int SEGS = Geo<FMT>::SEGS;
  // BF16 rows are twice as wide: a single wave gathers them in two register
  // batches at tile time instead of prefetching them
  constexpr int NB = (FMT == DSA_LAT_BF16 && NW == 1) ? 2 : 1;
  constexpr int SPT = (SEGS + NW * NB - 1) / (NW * NB);
  __shared__ __attribute__((aligned(16))) __bf16 lat[kRT * kLPad];
  __shared__ float rsc[kRT];
  __shared__ int rv[kRT];          // row id of the tile in LDS, -1 = absent
  __shared__ int ridbuf[2][kRT];   // row ids of the next two tiles

  const int split = blockIdx.x, t = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, ht = blockIdx.z * NW + wave;
  const int g = lane >> 4, c = lane & 15;
  const int my_row = lane >> 2, q = lane & 3;
  const int j_begin = split * p.split_len;
  const int j_end = min(j_begin + p.split_len, p.k);
  const int ntile = (j_end - j_begin + kRT - 1) / kRT;
  const int P = 1 << p.plog2;
  const int32_t* rlist = p.rows + (int64_t)t * p.k;
  auto load_id = [&](int tile) -> int {
    const int j = j_begin + tile * kRT + tid;
    return (tid < kRT && tile < ntile && j < j_end) ? rlist[j] : -1;
  };
  // FP8 row scale, fetched by the lane that owns chunk 0 of the row in wave 0
  const bool scale_lane = (FMT == DSA_LAT_FP8) && wave == 0 && q == 0;
  auto load_scale = [&](int id) -> float {
    if (!row_ok(id, p)) return 0.f;
    return *reinterpret_cast<const float*>(row_ptr<FMT>(p, id, P).data + LatRow<DSA_LAT_FP8>::kScale);
  };

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

  // pipeline prologue: ids of tiles 0 and 1, loads of tile 0, ids of tile 2
  if (tid < kRT) {
    ridbuf[0][tid] = load_id(0);
    ridbuf[1][tid] = load_id(1);
  }
  __syncthreads();
  i32x4 raw[SPT];
  uint32_t aux[SPT];
  float sc_next = 0.f;
  if (NB == 1) {
    const int id = ridbuf[0][my_row];
    seg_load<FMT, NW, SPT>(row_ptr<FMT>(p, id, P), wave, q, raw, aux);
    if (scale_lane) sc_next = load_scale(id);
  }
  int id_next = load_id(2);
  __bf16* lrow = lat + my_row * kLPad;

  for (int it = 0; it < ntile; ++it) {
    __syncthreads();  // the previous tile's readers are done with lat/rsc/rv
    // stage A: tile `it` (in registers) -> LDS
    if (NB == 1) {
      seg_store<FMT, NW, SPT>(lrow, wave, q, raw, aux);
    } else {
      const RowPtr rp = row_ptr<FMT>(p, ridbuf[it & 1][my_row], P);
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        seg_load<FMT, NW * NB, SPT>(rp, wave + b * NW, q, raw, aux);
        seg_store<FMT, NW * NB, SPT>(lrow, wave + b * NW, q, raw, aux);
      }
    }
    if (tid < kRT) {
      const int id = ridbuf[it & 1][tid];
      rv[tid] = row_ok(id, p) ? id : -1;
      if (FMT != DSA_LAT_FP8) rsc[tid] = row_ok(id, p) ? 1.f : 0.f;
    }
    if (scale_lane) rsc[my_row] = sc_next;
    __syncthreads();
    if (tid < kRT) ridbuf[it & 1][tid] = id_next;  // ids of tile it+2 (tile it's ids are consumed)
    // stage B: loads of tile it+1 stay in flight while tile `it` computes
    if (NB == 1 && it + 1 < ntile) {
      const int id = ridbuf[(it + 1) & 1][my_row];
      seg_load<FMT, NW, SPT>(row_ptr<FMT>(p, id, P), wave, q, raw, aux);
      if (scale_lane) sc_next = load_scale(id);
    }
    id_next = load_id(it + 3);
    mla_tile<8>(p, lat, rsc, rv, qf, O, m, l, g, c, 0);
  }

  mla_finish<8>(p, O, m, l, t, split, ht, g, c, 0);
}

// ---------------------------------------------------------------------------
// FP8 and NVFP4 latents: gather by direct HBM -> LDS copies.
//
// global_load_lds_dwordx4 writes each lane's 16 bytes straight into LDS (64
// lanes = 16 rows x 64 bytes per instruction), so DP tiles can be in flight
// behind the one being computed without holding a single register.  The
// split's row ids are read into LDS once, up front, so no copy ever waits on
// an id load.  The copies are issued from inline assembly and waited for with
// explicit vmcnt counts: every wave issues the same sequence per tile (one
// side copy -- FP8 row scales or NVFP4 block scales -- and its segment
// copies), always, even past the end of the list (rows on the zero row), so
// one constant count is exact in every iteration.
//
// Per iteration `it`, for every wave:
//   wait   copies of tile it (rows, side) have landed
//   A      dequantise this wave's segments of tile it into the bf16 tile
//   B      copy side and rows of tile it+DP into the ring slot tile it vacated
//   C      QK / softmax / PV of tile it
// LDS: bf16 tile [16][kLPad] | raw [DP][SEGS][1 KB] | side [DP][1 KB] | ids [split_len]
static __device__ __attribute__((aligned(64))) uint8_t g_zero_row[1280] = {0};

constexpr int kMlaDepth = 2;  // tiles in flight behind the one being computed
inline size_t mla_dma_lds_bytes(int segs, int depth, int split_len) {
  return (size_t)kRT * kLPad * 2 + (size_t)depth * (segs * 1024 + 1024) + ((size_t)split_len * 4 + 15) / 16 * 16;
}

// Direct HBM -> LDS copies.  NT = true sets the nontemporal hint: decode
// gathers rows no other workgroup reads again, and cached copies would also
// pay for evicting whatever dirty lines the caches hold (measured: 103 -> 72
// us on the 64K speculative batch); prefill rows are gathered by many query
// rows of the same request and keep the default, caching, policy.
template <bool NT>
__device__ __forceinline__ void dma16(const void* src, uint32_t lds) {
  if (NT) asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off nt" : : "v"(src), "s"(lds) : "memory", "m0");
  else asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "s"(lds) : "memory", "m0");
}
template <bool NT>
__device__ __forceinline__ void dma4(const void* src, uint32_t lds) {
  if (NT) asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off nt" : : "v"(src), "s"(lds) : "memory", "m0");
  else asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" : : "v"(src), "s"(lds) : "memory", "m0");
}
template <int N> __device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

template <int FMT> struct DmaGeo;
template <> struct DmaGeo<DSA_LAT_FP8> { static constexpr int SEGS = 9; };    // 576 B of E4M3
template <> struct DmaGeo<DSA_LAT_NVFP4> { static constexpr int SEGS = 5; };  // 256 B codes, 64 B rope

// Workgroup = NW head tiles, one wave each; DP tiles of rows in flight.
template <int FMT, int NW, int DP, int VS>
__global__ __launch_bounds__(64 * NW, VS) void mla_dma_kernel(MlaParams p) {
  constexpr int NA = 8 / VS;  // 64-dim value blocks per wave
  constexpr int SEGS = DmaGeo<FMT>::SEGS;
  constexpr int SPT = (SEGS + NW - 1) / NW;  // segment copies per wave per tile
  constexpr int kRawBytes = SEGS * 1024;
  extern __shared__ __attribute__((aligned(16))) uint8_t dsm[];
  __bf16* lat = reinterpret_cast<__bf16*>(dsm);
  uint8_t* raw = dsm + kRT * kLPad * 2;      // [DP][SEGS][1024]
  uint8_t* side = raw + DP * kRawBytes;      // [DP][1024]
  int* ids = reinterpret_cast<int*>(side + DP * 1024);  // [split_len]
  __shared__ float rsc[kRT];
  __shared__ int rv[kRT];

  const int split = blockIdx.x, t = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = NW == 1 ? 0 : __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ht = blockIdx.z * (NW / VS) + wave / VS;
  const int a0 = (wave % VS) * NA;  // first value block of this wave
  const int g = lane >> 4, c = lane & 15;
  const int my_row = lane >> 2, q = lane & 3;
  const int j_begin = split * p.split_len;
  const int j_end = min(j_begin + p.split_len, p.k);
  const int ntile = (j_end - j_begin + kRT - 1) / kRT;
  const int P = 1 << p.plog2;
  const int32_t* rlist = p.rows + (int64_t)t * p.k;
  const int n_ids = j_end - j_begin;  // >= 1
  const uint32_t raw_l = lds_addr(raw), side_l = lds_addr(side);

  // id of row r of tile `tile` (-1 past the split's end)
  auto id_at = [&](int tile, int r) -> int {
    const int j = tile * kRT + r;
    const int v = ids[min(j, n_ids - 1)];
    return j < n_ids ? v : -1;
  };
  auto row_of = [&](int id) -> const uint8_t* {
    return p.lat + (int64_t)(id >> p.plog2) * p.page_bytes + (int64_t)(id & (P - 1)) * LatRow<FMT>::kBytes;
  };
  // side and row copies of one tile into ring slot `slot`
  auto copy_tile = [&](int tile, int slot) {
    if (FMT == DSA_LAT_FP8) {
      // row scale of row lane >> 2 (lanes 4r .. 4r+3 carry row r's)
      const int id = id_at(tile, my_row);
      const uint8_t* src = row_ok(id, p) ? row_of(id) + LatRow<FMT>::kScale : g_zero_row;
      dma4<true>(src, side_l + slot * 1024);
    } else {
      // 32 bytes of E4M3 block scales per row: lane l < 32 copies half l & 1
      // of row l >> 1 (lanes 32..63 repeat rows 0..15 into the slot's tail)
      const int r = (lane >> 1) & 15;
      const int id = id_at(tile, r);
      const uint8_t* src = row_ok(id, p) ? row_of(id) + LatRow<FMT>::kScales + (lane & 1) * 16 : g_zero_row;
      dma16<true>(src, side_l + slot * 1024);
    }
    const int id = id_at(tile, my_row);
    // an absent row reads the zero row (never past its 1280 bytes)
    const uint8_t* row = row_ok(id, p) ? row_of(id) : g_zero_row;
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      const int sp = min(wave + i * NW, SEGS - 1);
      // FP8: 9 segments of 64 codes; NVFP4: 4 segments of codes, then the rope
      const int off = (FMT == DSA_LAT_NVFP4 && sp == 4) ? LatRow<FMT>::kRope : sp * 64;
      dma16<true>(row + off + q * 16, raw_l + slot * kRawBytes + sp * 1024);
    }
  };
  // copies still outstanding (tiles it+1 .. it+DP-1) when tile it is consumed
  constexpr int kBehind = (DP - 1) * (1 + SPT);
  static_assert(kBehind < 64, "vmcnt range");

  // the split's row ids, read once (plain loads; waited for by the compiler)
  for (int j = tid; j < n_ids; j += 64 * NW) ids[j] = rlist[j_begin + j];

  bf16x8 qf[18];
  {
    const int head = 16 * ht + c;
    if (head < p.H) {
      const __bf16* qp = p.q + ((int64_t)t * p.H + head) * 576;
#pragma unroll
      for (int kk = 0; kk < 18; ++kk) qf[kk] = __builtin_bit_cast(bf16x8, ld16(qp + dim_of(kk, g)));
    } else {
#pragma unroll
      for (int kk = 0; kk < 18; ++kk) qf[kk] = bf16x8{};
    }
  }
  f32x4 O[NA * 4];
#pragma unroll
  for (int x = 0; x < NA * 4; ++x) O[x] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -__builtin_inff(), l = 0.f;

  // The query loads must be complete (and known to the compiler to be) before
  // the first copy: the compiler does not see the copies, and a query load
  // still pending at the loop would make it wait for everything in flight.
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();                     // ids visible to every wave
  // prologue: tiles 0 .. DP-1
#pragma unroll
  for (int d = 0; d < DP; ++d) copy_tile(d, d);
  __bf16* lrow = lat + my_row * kLPad;

  for (int it = 0; it < ntile; ++it) {
    const int slot = it % DP;
    wait_vmcnt<kBehind>();
    __syncthreads();  // the previous tile's readers are done with lat/rsc/rv
    // A: this wave's segments of tile `it` -> bf16 tile (all LDS reads are
    // issued before the first store, which the compiler could not reorder)
    i32x4 rseg[SPT];
    uint32_t rsc2[SPT];
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      const int sp = min(wave + i * NW, SEGS - 1);
      rseg[i] = *reinterpret_cast<const i32x4*>(raw + slot * kRawBytes + sp * 1024 + lane * 16);
      rsc2[i] = FMT == DSA_LAT_NVFP4
                    ? *reinterpret_cast<const uint16_t*>(side + slot * 1024 + my_row * 32 + (min(sp, 3) * 4 + q) * 2)
                    : 0u;
    }
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      const int sp = wave + i * NW;
      if (sp >= SEGS) continue;
      const i32x4 v = rseg[i];
      if (FMT == DSA_LAT_FP8 || sp == 4) {
        const i32x2 a = e4m3x4_to_bf16(v[0]), b = e4m3x4_to_bf16(v[1]);
        const i32x2 c2 = e4m3x4_to_bf16(v[2]), d = e4m3x4_to_bf16(v[3]);
        i32x4* dst = reinterpret_cast<i32x4*>(lrow + (FMT == DSA_LAT_FP8 ? (sp * 4 + q) * 16 : 512 + q * 16));
        dst[0] = i32x4{a[0], a[1], b[0], b[1]};
        dst[1] = i32x4{c2[0], c2[1], d[0], d[1]};
      } else {  // NVFP4 codes: 32 dims, two E4M3 block scales
        const uint32_t sc2 = rsc2[i];
        const float sa = e4m3_to_f32(sc2 & 0xFFu), sb = e4m3_to_f32((sc2 >> 8) & 0xFFu);
        i32x4* dst = reinterpret_cast<i32x4*>(lrow + (sp * 4 + q) * 32);
        dst[0] = __builtin_bit_cast(i32x4, e2m1x8_times(v[0], sa));
        dst[1] = __builtin_bit_cast(i32x4, e2m1x8_times(v[1], sa));
        dst[2] = __builtin_bit_cast(i32x4, e2m1x8_times(v[2], sb));
        dst[3] = __builtin_bit_cast(i32x4, e2m1x8_times(v[3], sb));
      }
    }
    if (wave == 0 && tid < kRT) {
      const int id = id_at(it, tid);
      const bool ok = row_ok(id, p);
      rv[tid] = ok ? id : -1;
      rsc[tid] = FMT == DSA_LAT_FP8 ? *reinterpret_cast<const float*>(side + slot * 1024 + tid * 16)
                                    : (ok ? 1.f : 0.f);
    }
    __syncthreads();
    // B: tile it+DP into the slot tile it vacated
    copy_tile(it + DP, slot);
    // C
    mla_tile<NA>(p, lat, rsc, rv, qf, O, m, l, g, c, a0);
  }
  wait_vmcnt<0>();  // no copy may land after the workgroup's LDS is released
  mla_finish<NA>(p, O, m, l, t, split, ht, g, c, a0);
}

// ---------------------------------------------------------------------------
// Prefill over FP8 latents: 16-row tiles computed straight from a small copy
// ring.  (Decode keeps mla_dma_kernel: there the row gather, not the tile
// chain, bounds the time, and its deeper copy ring with nontemporal copies
// gathers faster: 72 against 88 us on the 64K speculative batch.)
//
// No BF16 copy of a tile is made: the copies land in LDS in the order the
// MFMA operands want them and every wave converts the FP8 codes it needs in
// registers (exact: E4M3 -> BF16).  A workgroup needs under 20 KB of LDS (two
// ring slots and a ring of row ids), so eight one-wave workgroups share a CU:
// two waves per SIMD, whose MFMA and VALU work interleave (one wave per SIMD
// leaves every instruction waiting on its predecessor's latency).
//
// Ring slot (one tile): 9 segments of 1 KB and the 16 FP8 row scales.  Copy
// instruction sp: lane L = 16 j + r copies bytes 64 sp + 16 j .. +15 of row r
// to slot offset sp * 1024 + 16 L.  The row ids come through a ring of their
// own (one 4-byte copy per lane, three tiles ahead), so no copy address ever
// waits on an id load and the list need not be staged whole.
//   QK  S^T[rows x heads] on v_mfma_f32_16x16x32_bf16: k-step kk (< 18) of
//       lane (g, c) covers dims 64 (kk/2) + 16 g + 8 (kk%2) .. +7 of latent row
//       c (its own copy position, 16 bytes for two k-steps) and of head c;
//       lane (g, c) gets rows 4g+i of head c.
//   PV  O[heads x 512] += P[heads x 16] . V[16 x 512] on
//       v_mfma_f32_16x16x16_bf16 (A: the weights of rows 4g+i, in the lanes
//       that computed them).  One transposing byte read (ds_read_b64_tr_b8:
//       result lane c, byte j is byte c%8 of the 8 bytes source lane 2j + c/8
//       points at) gives every lane rows 4g..4g+3 of two dims, d0 + c (bytes
//       0-3) and d0 + 16 + c (bytes 4-7): the V operands of two MFMAs.
// The per-row FP8 scale multiplies the logit and the softmax weight.
constexpr int kXcds = 8;  // MI355X: eight XCDs, each with its own L2
constexpr int kF8ScaleOff = 9 * 1024;
constexpr int kF8Slot = kF8ScaleOff + 256;
constexpr int kF8Copies = 9 + 1;               // copies per tile: 9 segments, the row scales
// DP ring slots (tiles it+1 .. it+DP-1 in flight while tile it computes) and
// 2 DP id slots (ids run DP tiles ahead of the copies that need them)
constexpr int mla_f8_lds(int dp) { return dp * kF8Slot + 2 * dp * 256; }
static_assert(mla_f8_lds(2) <= 160 * 1024 / 8, "one-wave workgroups: eight per CU");
static_assert(mla_f8_lds(4) <= 160 * 1024 / 4, "two-wave workgroups: four per CU");

template <int NW, int DP>
__global__ __launch_bounds__(64 * NW) void mla_f8_kernel(MlaParams p) {
  constexpr int kPer = (kF8Copies + NW - 1) / NW;  // copies per wave per tile (the last one repeated)
  constexpr int kIdSlots = 2 * DP;
  constexpr int kBehind = (DP - 1) * (1 + kPer);   // this wave's ops issued after tile it's copies
  static_assert(kBehind < 64 && DP * (1 + kPer) < 64, "vmcnt range");
  __shared__ __attribute__((aligned(16))) uint8_t ring[mla_f8_lds(DP)];
  uint8_t* idr = ring + DP * kF8Slot;  // [kIdSlots][64 ints]

  // XCD-aware order (one split per row): workgroups go to the eight XCDs
  // round-robin by linear id, so the `groups` workgroups of a query row get
  // ids 8 apart -- one XCD, dispatched back to back -- and the second and
  // later ones find the row's latents in that XCD's L2.
  const int groups = gridDim.x / ((p.T + kXcds - 1) / kXcds * kXcds);
  const int lin = blockIdx.x, xcd = lin % kXcds, slot_x = lin / kXcds;
  const int split = 0, t = (slot_x / groups) * kXcds + xcd, grp = slot_x % groups;
  if (t >= p.T) return;  // padding of the last XCD round (the whole workgroup leaves)
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = NW == 1 ? 0 : __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ht = grp * NW + wave;
  const bool active = ht < p.ntiles;  // a wave past the last head tile only copies
  const int g = lane >> 4, c = lane & 15;
  const int j_begin = split * p.split_len;
  const int n_ids = min(j_begin + p.split_len, p.k) - j_begin;  // >= 1
  const int ntile = (n_ids + kRT - 1) / kRT;
  const int P = 1 << p.plog2;
  const int32_t* rlist = p.rows + (int64_t)t * p.k + j_begin;
  const uint32_t ring_l = lds_addr(ring), idr_l = lds_addr(idr);

  // id copy of tile `tile` (every wave issues it: identical bytes)
  auto copy_ids = [&](int tile) {
    dma4<false>(rlist + min(tile * kRT + c, n_ids - 1), idr_l + (tile % kIdSlots) * 256);
  };
  // id of row r of a tile whose ids have landed (-1 past the split's end)
  auto id_at = [&](int tile, int r) -> int {
    const int v = reinterpret_cast<const int*>(idr + (tile % kIdSlots) * 256)[r];
    return tile * kRT + r < n_ids ? v : -1;
  };
  auto row_of = [&](int id) -> const uint8_t* {
    return row_ok(id, p) ? p.lat + (int64_t)(id >> p.plog2) * p.page_bytes + (int64_t)(id & (P - 1)) * 640
                         : g_zero_row;
  };
  // this wave's copies of a tile (source row `row`, this lane's) into ring
  // slot `slot`: kPer of them whatever the tile, so one vmcnt count is exact
  auto copy_tile = [&](const uint8_t* row, int slot) {
    const uint32_t base = ring_l + slot * kF8Slot;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int x = min(wave + i * NW, kF8Copies - 1);  // uniform
      if (x < 9) dma16<false>(row + 64 * x + 16 * g, base + x * 1024);
      else dma4<false>(row + 576, base + kF8ScaleOff);
    }
  };

  // query fragments of head 16 ht + c in the k-step order above
  bf16x8 qf[18];
  {
    const int head = 16 * ht + c;
    if (active && head < p.H) {
      const __bf16* qp = p.q + ((int64_t)t * p.H + head) * 576 + 16 * g;
#pragma unroll
      for (int kk = 0; kk < 18; ++kk) qf[kk] = __builtin_bit_cast(bf16x8, ld16(qp + 64 * (kk >> 1) + 8 * (kk & 1)));
    } else {
#pragma unroll
      for (int kk = 0; kk < 18; ++kk) qf[kk] = bf16x8{};
    }
  }
  f32x4 O[32];
#pragma unroll
  for (int x = 0; x < 32; ++x) O[x] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -__builtin_inff(), l = 0.f;

  // Prologue: ids(0 .. DP-1), all landed; then [ids(d + DP), copies(d)] for
  // d < DP; at the end of every tile it: [ids(it + 2 DP), copies(it + DP)].
  // The ids a copy needs were issued just before the copies of DP tiles
  // earlier, which have landed by then.
#pragma unroll
  for (int d = 0; d < DP; ++d) copy_ids(d);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the ids and (seen by the compiler) the query loads
#pragma unroll
  for (int d = 0; d < DP; ++d) {
    copy_ids(d + DP);
    copy_tile(row_of(id_at(d, c)), d);
  }


  for (int it = 0; it < ntile; ++it) {
    const int slot = it % DP;
    wait_vmcnt<kBehind>();  // this wave's copies of tile `it` (later ids and copies may fly)
    __syncthreads();        // ... and every other wave's
    const uint8_t* sl = ring + slot * kF8Slot;
    // the source row of this lane's next copies (tile it+DP), ahead of the
    // products so that its id read and address are ready when they are issued
    const uint8_t* next_row = row_of(id_at(it + DP, c));
    if (active) {
      // the tile's row scales and ids, read before the products
      const f32x4 sc = *reinterpret_cast<const f32x4*>(sl + kF8ScaleOff + 16 * g);
      bool ok[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) ok[i] = row_ok(id_at(it, 4 * g + i), p);
      // ---- QK: one accumulator chain (an MFMA that accumulates into the
      // previous one's result issues behind it; the second wave per SIMD
      // fills the gaps, and no partial sums need adding)
      f32x4 s = {0.f, 0.f, 0.f, 0.f};
      {
        const uint8_t* src = sl + lane * 16;
#pragma unroll
        for (int sp = 0; sp < 9; ++sp) {
          const i32x4 raw = *reinterpret_cast<const i32x4*>(src + sp * 1024);
          s = mfma16x16x32(e4m3x8_to_bf16x8(raw[0], raw[1]), qf[2 * sp], s);
          s = mfma16x16x32(e4m3x8_to_bf16x8(raw[2], raw[3]), qf[2 * sp + 1], s);
        }
      }
      // ---- online softmax for head c over rows 4g+i
      float lg[4];
      float tmax = -__builtin_inff();
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float v = ok[i] ? s[i] * p.sm_log2 * sc[i] : -__builtin_inff();
        lg[i] = v;
        tmax = fmaxf(tmax, v);
      }
      tmax = fmaxf(tmax, xor16(tmax, g));
      tmax = fmaxf(tmax, xor32(tmax, g));
      const float mnew = (m == -__builtin_inff() || tmax > m + kRescaleLog2) ? tmax : m;
      const float alpha = (m == -__builtin_inff()) ? 1.f : exp2_hw(m - mnew);
      // a finite floor for the max: a -inf logit then weighs 2^-inf = 0 even
      // while every logit so far is -inf
      const float mref = fmaxf(mnew, -3.0e38f);
      float psum = 0.f, pw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e = exp2_hw(lg[i] - mref);
        psum += e;
        pw[i] = e * sc[i];
      }
      psum += xor16(psum, g);
      psum += xor32(psum, g);
      l = l * alpha + psum;
      m = mnew;
      const i32x2 pa2 = {(int)pack_bf16x2(pw[0], pw[1]), (int)pack_bf16x2(pw[2], pw[3])};
      const bf16x4 pa = __builtin_bit_cast(bf16x4, pa2);
      if (__ballot(alpha != 1.f)) {
        float ai[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) ai[i] = __shfl(alpha, 4 * g + i);
#pragma unroll
        for (int x = 0; x < 32; ++x)
#pragma unroll
          for (int i = 0; i < 4; ++i) O[x][i] *= ai[i];
      }
      // ---- PV: read n covers dims 32 n + c (O[2n]) and 32 n + 16 + c (O[2n+1])
      // transposed-read source of this lane: byte slot j = (lane%16)/2 -> row
      // 4g + j%4 of dim chunk j/4 (+16 dims), half lane%2 of the 16 bytes
      // (the lane id comes from an asm the compiler cannot hoist, so the
      // read offset is formed here each tile: kept live through the loop it
      // is the value spilled at 256 VGPRs)
      int ln;
      asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
      const int tj = (ln & 15) >> 1;
      const uint8_t* vsrc = sl + (tj >> 2) * 256 + (4 * (ln >> 4) + (tj & 3)) * 16 + 8 * (ln & 1);
#pragma unroll
      for (int n = 0; n < 16; ++n) {
        typedef int v2i __attribute__((ext_vector_type(2)));
        const auto* a = (const __attribute__((address_space(3))) v2i*)(const void*)(vsrc + (n >> 1) * 1024 +
                                                                                   (n & 1) * 512);
        const v2i vb = __builtin_amdgcn_ds_read_tr8_b64_v2i32(const_cast<__attribute__((address_space(3))) v2i*>(a));
        O[2 * n] = mfma16x16x16(pa, __builtin_bit_cast(bf16x4, e4m3x4_to_bf16((uint32_t)vb[0])), O[2 * n]);
        O[2 * n + 1] = mfma16x16x16(pa, __builtin_bit_cast(bf16x4, e4m3x4_to_bf16((uint32_t)vb[1])), O[2 * n + 1]);
      }
    }
    __syncthreads();  // every wave is done with the slot and with the ids of tile it
    copy_ids(it + 2 * DP);
    copy_tile(next_row, slot);
  }
  wait_vmcnt<0>();  // no copy may land after the workgroup's LDS is released
  if (active) mla_finish<8>(p, O, m, l, t, split, ht, g, c, 0);
}

// Merge of the split partials of one (row, head): all split LSEs are read in
// parallel, and the weighted sum over splits issues its loads back to back.
__global__ __launch_bounds__(128) void mla_combine_kernel(MlaParams p) {
  __shared__ float wsh[64];
  __shared__ float red[2];
  const int h = blockIdx.x, t = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ns = p.nsplit;  // <= 64
  const float* pl = p.part_lse + (int64_t)t * ns * p.H + h;
  const float ls = tid < ns ? pl[(int64_t)tid * p.H] : -__builtin_inff();
  float mx = ls;
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  mx = fmaxf(red[0], red[1]);
  const float w = (ls == -__builtin_inff()) ? 0.f : __expf(ls - mx);
  if (tid < 64) wsh[tid] = w;
  float ws = w;  // all ns <= 64 weights live in wave 0
  for (int o = 32; o > 0; o >>= 1) ws += __shfl_xor(ws, o);
  __syncthreads();
  if (tid == 0) red[0] = ws;
  __syncthreads();
  const float tot = red[0];
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if (mx != -__builtin_inff()) {
    const float* po = p.part_o + ((int64_t)t * ns * p.H + h) * 512 + 4 * tid;
#pragma unroll 8
    for (int s2 = 0; s2 < ns; ++s2) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(po + (int64_t)s2 * p.H * 512);
      acc += wsh[s2] * v;
    }
  }
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
  *reinterpret_cast<f32x4*>(p.out + ((int64_t)t * p.H + h) * 512 + 4 * tid) = acc * inv;
  if (tid == 0 && p.lse) p.lse[(int64_t)t * p.H + h] = tot > 0.f ? mx + __logf(tot) : -__builtin_inff();
}

// Scratch of the allocation-free decode entry point: the split partials of
// one call live in this file-scope device array (one copy per GPU, held until
// the process ends) instead of a caller workspace.  Host code never uses the
// array's name as an address: its device address is resolved once per device
// with hipGetSymbolAddress and kept.
static __device__ __align__(256) uint8_t scratch[kMlaScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

dsa_status mla_scratch(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DSA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* a = nullptr;
    if (hipGetSymbolAddress(&a, HIP_SYMBOL(scratch)) != hipSuccess || !a) return DSA_ERR_HIP;
    g_scratch_ptr[dev] = a;
  }
  *ptr = g_scratch_ptr[dev];
  return DSA_OK;
}

dsa_status launch_mla(const MlaParams& p, hipStream_t stream) {
  const MlaShape sh = mla_shape(p.ntiles, p.fmt == DSA_LAT_NVFP4);
  dim3 grid(p.nsplit, p.T, sh.groups), block(64 * sh.nw);
#define DSA_MLA_LAUNCH(F)                                                                   \
  switch (sh.nw) {                                                                         \
    case 1: hipLaunchKernelGGL((mla_kernel<F, 1>), grid, block, 0, stream, p); break;      \
    case 2: hipLaunchKernelGGL((mla_kernel<F, 2>), grid, block, 0, stream, p); break;      \
    case 3: hipLaunchKernelGGL((mla_kernel<F, 3>), grid, block, 0, stream, p); break;      \
    default: hipLaunchKernelGGL((mla_kernel<F, 4>), grid, block, 0, stream, p); break;     \
  }
#define DSA_MLA_DMA_LAUNCH(F)                                                                         \
  {                                                                                                  \
    constexpr int DP = kMlaDepth;                                                                    \
    const size_t lds = mla_dma_lds_bytes(DmaGeo<F>::SEGS, DP, p.split_len);                          \
    if (sh.vs == 2) {                                                                                \
      hipLaunchKernelGGL((mla_dma_kernel<F, 2, DP, 2>), grid, block, lds, stream, p);                \
    } else {                                                                                         \
      switch (sh.nw) {                                                                               \
        case 1: hipLaunchKernelGGL((mla_dma_kernel<F, 1, DP, 1>), grid, block, lds, stream, p); break; \
        case 2: hipLaunchKernelGGL((mla_dma_kernel<F, 2, DP, 1>), grid, block, lds, stream, p); break; \
        case 3: hipLaunchKernelGGL((mla_dma_kernel<F, 3, DP, 1>), grid, block, lds, stream, p); break; \
        default: hipLaunchKernelGGL((mla_dma_kernel<F, 4, DP, 1>), grid, block, lds, stream, p); break; \
      }                                                                                              \
    }                                                                                                \
  }
  switch (p.fmt) {
    case DSA_LAT_BF16: DSA_MLA_LAUNCH(DSA_LAT_BF16) break;
    case DSA_LAT_FP8: {
      if (!p.prefill) {
        DSA_MLA_DMA_LAUNCH(DSA_LAT_FP8)
        break;
      }
      const MlaShape s8 = mla_shape_fp8(p.ntiles);
      // one split per row (prefill): a 1-D grid in the XCD-aware order
      const dim3 g8((p.T + kXcds - 1) / kXcds * kXcds * s8.groups), b8(64 * s8.nw);
      // ring depth: all the LDS a CU's eight waves leave (two slots per one-wave
      // workgroup, four per two-wave one)
      switch (s8.nw) {
        case 1: hipLaunchKernelGGL((mla_f8_kernel<1, 2>), g8, b8, 0, stream, p); break;
        case 2: hipLaunchKernelGGL((mla_f8_kernel<2, 4>), g8, b8, 0, stream, p); break;
        default: hipLaunchKernelGGL((mla_f8_kernel<4, 4>), g8, b8, 0, stream, p); break;
      }
      break;
    }
    default: DSA_MLA_DMA_LAUNCH(DSA_LAT_NVFP4) break;
  }
#undef DSA_MLA_LAUNCH
#undef DSA_MLA_DMA_LAUNCH
  if (p.nsplit > 1) hipLaunchKernelGGL(mla_combine_kernel, dim3(p.H, p.T), dim3(128), 0, stream, p);
  return hipGetLastError() == hipSuccess ? DSA_OK : DSA_ERR_HIP;
}

DSA_DEBUG_TAKE(mla)

}  // namespace dsa
