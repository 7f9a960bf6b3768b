// Lightning indexer, decode shape: BF16 queries against FP8, MXFP4 or NVFP4
// paged keys.
//
//   score(t, s) = sum_{h<32} w[t,h] * max(0, q[t,h,:] . k_s)
//
// (Kimi K3.1 Pro day-0 page, "Sparse attention in K3.1 Pro": 32 light heads
// score every earlier token against a 132-byte FP8 key; AMD section "native
// MXFP4 indexer": FP32 accumulation, weighted reduction across heads, keys
// reused across the speculative query rows of a request.  MiniMax-M3.1-Flash
// day-0 page, "Quick start" and AMD "NVFP4 indexer DCP": NVFP4 index keys,
// E2M1 with one E4M3 scale per 16 dims.)
//
// Work split: one workgroup = one request x one chunk of keys.  The rows of
// the request (q, 8 KiB each as bf16) are staged once in LDS; each wave streams
// its share of the chunk's keys with 16-byte loads straight into MFMA
// B-fragments (dequantised in registers, exactly, to bf16), and runs every row
// against them on v_mfma_f32_16x16x32_bf16.  Keys are therefore read from HBM
// once per request whatever the number of rows.
//
// Fragment layout (16 keys x 32 heads per MFMA pair): lane l = 16*g + c holds
// key c of the tile and, for k-step kk (0..3), dims 32g + 8kk .. +7.  The A
// operand (q) uses the same dim assignment for head c (+16 for the second
// head tile), so the k-sum is the full 128-dim dot product.  The result lane
// (g, c) holds heads 4g+i (i<4) for key c; the ReLU-weighted head sum is done
// in-lane, then a reduce-scatter over the four lane groups (three cross-row
// swaps for four tiles) leaves every lane with one finished score, and the
// wave stores 64 consecutive scores.
#include "common.h"
#include "kernels.h"

namespace dsa {

constexpr int kIdxWaves = 4;
constexpr int kIdxKT = 4;              // 16-key tiles per wave per round
constexpr int kIdxRound = kIdxWaves * kIdxKT * 16;  // 256 keys per round
constexpr int kQPad = 136;             // bf16 per head row in LDS (272 B: conflict-free reads)
constexpr int kQ8Pad = 144;            // bytes per FP8 head row in LDS (conflict-free 16-byte reads)

// Raw key bytes of one round (kIdxKT tiles of 16 keys) for one lane: the
// codes of the lane's 32 dims of key c of each tile and their side data.
template <int KFMT> struct RawKeys {
  i32x4 v[kIdxKT][KFMT == DSA_KEY_FP8 ? 2 : 1];
  bool ok[kIdxKT];       // page present and tile inside the chunk
  uint32_t sc[kIdxKT];   // (side data read in the loop) MXFP4: E8M0 codes of key c of tile kt;
                         // NVFP4: the two E4M3 block scales of this lane's 32 dims
  float own_scale;       // (side data read in the loop) FP8 scale of the key this lane stores
};

// The 8 dims lane group g supplies at k-step kk of the 128-dim dot product
// (the same assignment for the query A and the key B fragments, so the
// k-sum is the full dot product).  FP8 keys: the four lane groups of a key
// read its first 64 bytes in one instruction and its last 64 in a second
// (16 bytes each, contiguous per key); MXFP4: lane group g holds the 32
// codes under E8M0 scale g; NVFP4: the same 32 codes under block scales 2g
// and 2g+1.
// (COAL = false: FP8 lane group g reads bytes 32g .. 32g+31 of each key, as
// the multi-row kernel does, whose A fragments come from LDS.)
template <int KFMT, bool COAL>
__device__ __forceinline__ int kdim(int kk, int g) {
  if (KFMT == DSA_KEY_FP8 && COAL) return kk < 2 ? 16 * g + 8 * kk : 64 + 16 * g + 8 * (kk - 2);
  return 32 * g + 8 * kk;
}

// Page ids of the chunk's logical pages, staged in LDS once per workgroup so a
// round's key loads never wait on a block-table load.
constexpr int kIdxMaxChunkPages = 4096 / 16 + 1;
constexpr int kIdxMaxRows = kIndexerMaxRowsPerPass;  // rows staged in LDS per pass (qrows)

// Key loads carry the nontemporal hint (each key byte is used by one
// workgroup, once): measured 9% faster on the 64K speculative batch after an
// L2/MALL scrub, where cached loads also paid for evicting the scrub's dirty
// lines.  Every load is issued unconditionally (a tile past the chunk end or on an
// absent page reads page 0 instead and its scores are masked afterwards):
// loads under a branch would make the compiler wait for all of them before
// any is used, so the next round's loads could not overlap this round.
template <int KFMT>
__device__ __forceinline__ void load_round(const IndexerParams& p, const int* pg_lds, int lp0, int base, int kend,
                                           int wave, int g, int c, int P, RawKeys<KFMT>& raw) {
  const int last = ((kend - 1) >> p.plog2) - lp0;  // last staged page entry
  int pgs[kIdxKT];
#pragma unroll
  for (int kt = 0; kt < kIdxKT; ++kt) {
    const int s0 = base + (wave * kIdxKT + kt) * 16;
    const int e = min((s0 >> p.plog2) - lp0, last);
    // read unconditionally (e is clamped to a staged entry): a read under a
    // branch would make each tile wait for its page id before the next is read
    const int pg_read = pg_lds[e];
    const int pg = s0 < kend ? pg_read : -1;
    pgs[kt] = pg;
    raw.ok[kt] = pg >= 0;
    const uint8_t* page = p.keys + (int64_t)max(pg, 0) * p.page_bytes;
    const int slot = (s0 & (P - 1)) + c;
    if (KFMT == DSA_KEY_FP8) {
      const uint8_t* kp = page + slot * 128 + 32 * g;
      raw.v[kt][0] = ld16_stream(kp);
      raw.v[kt][KFMT == DSA_KEY_FP8 ? 1 : 0] = ld16_stream(kp + 16);
    } else if (KFMT == DSA_KEY_MXFP4) {
      raw.v[kt][0] = ld16_stream(page + slot * 64 + 16 * g);
      raw.sc[kt] = *reinterpret_cast<const uint32_t*>(page + P * 64 + slot * 4);
    } else {
      // NVFP4: dims 32g .. 32g+31 lie in blocks 2g and 2g+1, whose scales are
      // bytes 2g, 2g+1 of the key's eight
      raw.v[kt][0] = ld16_stream(page + slot * 64 + 16 * g);
      raw.sc[kt] = *reinterpret_cast<const uint16_t*>(page + P * 64 + slot * 8 + 2 * g);
    }
  }
  if (KFMT == DSA_KEY_FP8) {
    // one load for the scale of the key this lane stores (tile g, key c)
    int pg = pgs[0];
#pragma unroll
    for (int kt = 1; kt < kIdxKT; ++kt)
      if (g == kt) pg = pgs[kt];
    const int slot = ((base + (wave * kIdxKT + g) * 16) & (P - 1)) + c;
    raw.own_scale = __builtin_nontemporal_load(reinterpret_cast<const float*>(p.keys + (int64_t)max(pg, 0) * p.page_bytes + P * 128 + slot * 4));
  }
}

// Dequantise tile kt of a round into B fragments (exact in bf16).
template <int KFMT>
__device__ __forceinline__ void dequant_tile(const RawKeys<KFMT>& raw, int kt, bf16x8 (&b)[4], uint32_t e8m0x4 = 0,
                                             int g = 0) {
  if (KFMT == DSA_KEY_FP8) {
    const i32x4 x = raw.v[kt][0], y = raw.v[kt][KFMT == DSA_KEY_FP8 ? 1 : 0];
    b[0] = e4m3x8_to_bf16x8(x[0], x[1]);
    b[1] = e4m3x8_to_bf16x8(x[2], x[3]);
    b[2] = e4m3x8_to_bf16x8(y[0], y[1]);
    b[3] = e4m3x8_to_bf16x8(y[2], y[3]);
  } else if (KFMT == DSA_KEY_MXFP4) {
    const i32x4 x = raw.v[kt][0];
    const float sc = e8m0_to_f32((e8m0x4 >> (8 * g)) & 0xFFu);
    b[0] = e2m1x8_to_bf16x8(x[0], sc);
    b[1] = e2m1x8_to_bf16x8(x[1], sc);
    b[2] = e2m1x8_to_bf16x8(x[2], sc);
    b[3] = e2m1x8_to_bf16x8(x[3], sc);
  } else {
    // NVFP4: e8m0x4 holds this lane's two E4M3 block scales (dims 32g..+15,
    // 32g+16..+31); E2M1 x E4M3 is exact in bf16
    const i32x4 x = raw.v[kt][0];
    const float s0 = e4m3_to_f32(e8m0x4 & 0xFFu), s1 = e4m3_to_f32((e8m0x4 >> 8) & 0xFFu);
    b[0] = e2m1x8_times(x[0], s0);
    b[1] = e2m1x8_times(x[1], s0);
    b[2] = e2m1x8_times(x[2], s1);
    b[3] = e2m1x8_times(x[3], s1);
  }
}

// Multiplier of the score this lane stores (key s_own = tile g, key c): the
// FP8 key scale, 1 for MXFP4 / NVFP4 (whose block scales are applied exactly
// during dequantisation), or -inf on an absent page.  A tile on an absent page holds
// page 0's bytes; every score it produces is replaced by this -inf.
template <int KFMT>
__device__ __forceinline__ float own_multiplier(const RawKeys<KFMT>& raw, int g) {
  bool own_ok = raw.ok[0];
#pragma unroll
  for (int kt = 1; kt < kIdxKT; ++kt)
    if (g == kt) own_ok = raw.ok[kt];
  return own_ok ? (KFMT == DSA_KEY_FP8 ? raw.own_scale : 1.f) : -__builtin_inff();
}

// Q8: FP8 queries (codes + per-(row, head) scale, folded into the staged head
// weight) against FP8 keys on the FP8 matrix instruction: one
// v_mfma_scale_f32_16x16x128_f8f6f4 per 16 heads x 16 keys takes the raw key
// bytes the lane loaded (key c, bytes 32g .. 32g+31) as its B operand, so the
// keys are never converted.  (AMD section of the K3.1 page: the decode
// indexer on the 16x16x128 FP8 instruction.)
template <int KFMT, bool Q8>
__global__ __launch_bounds__(256, Q8 ? 3 : 1) void indexer_bf16_kernel(IndexerParams p) {
  // [rows][32][row bytes] queries (bf16, kQPad elements; or FP8, kQ8Pad bytes), then [rows][32] fp32 w
  extern __shared__ __attribute__((aligned(16))) uint8_t qsb[];
  static_assert(!Q8 || KFMT == DSA_KEY_FP8, "FP8 queries run against FP8 keys");
  constexpr int kRowB = Q8 ? kQ8Pad : kQPad * 2;  // LDS bytes per staged head
  __bf16* qs = reinterpret_cast<__bf16*>(qsb);
  __shared__ int s_vmax[kIdxWaves];
  __shared__ int s_vis[kIdxMaxRows];
  __shared__ int pg_lds[kIdxMaxChunkPages];

  const int r = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int rs = p.req_row_start[r], re = p.req_row_start[r + 1];
  float* ws = reinterpret_cast<float*>(qsb + p.qrows * 32 * kRowB);

  // Rows of a pass are staged with every load issued before the first LDS
  // store (one memory round trip, not one per load); the first pass's loads
  // are issued before the visible-range and page-table reads they do not
  // depend on.
  // 16-byte pieces per row: 512 (bf16: 16 per head) or 256 (FP8: 8 per head)
  constexpr int kPieceLog = Q8 ? 3 : 4;
  constexpr int kRowPieces = 32 << kPieceLog;
  constexpr int kQLoads = kIdxMaxRows * kRowPieces / 256;
  auto q_src = [&](int t, int head, int part) -> const void* {
    return Q8 ? (const void*)(p.q8 + ((int64_t)t * 32 + head) * 128 + part * 16)
              : (const void*)(p.q + ((int64_t)t * 32 + head) * 128 + part * 8);
  };
  auto q_dst = [&](int row, int head, int part) -> i32x4* {
    return reinterpret_cast<i32x4*>(qsb + (row * 32 + head) * kRowB + part * 16);
  };
  // staged head weight: w, times the FP8 query scale
  auto w_of = [&](int64_t th) -> float { return Q8 ? p.w[th] * p.q_scale[th] : p.w[th]; };
  i32x4 qv[kQLoads];
  float wv = 0.f;
  int vv = 0;
  auto load_rows = [&](int t0, int nr) {
#pragma unroll
    for (int u = 0; u < kQLoads; ++u) {
      const int i = tid + 256 * u;
      const int row = i >> (5 + kPieceLog), head = (i >> kPieceLog) & 31, part = i & ((1 << kPieceLog) - 1);
      if (i < nr * kRowPieces) qv[u] = ld16(q_src(t0 + row, head, part));
    }
    if (tid < nr * 32) wv = w_of((int64_t)t0 * 32 + tid);
    if (tid < nr) vv = clamp_vis(p.tok_vis[t0 + tid], p.max_vis);
  };
  auto store_rows = [&](int nr) {
#pragma unroll
    for (int u = 0; u < kQLoads; ++u) {
      const int i = tid + 256 * u;
      const int row = i >> (5 + kPieceLog), head = (i >> kPieceLog) & 31, part = i & ((1 << kPieceLog) - 1);
      if (i < nr * kRowPieces) *q_dst(row, head, part) = qv[u];
    }
    if (tid < nr * 32) ws[tid] = wv;
    // visible counts of the pass's rows, read from LDS in the row loop: a
    // global load there would make every row wait for the next round's keys
    if (tid < nr) s_vis[tid] = vv;
  };
  load_rows(rs, min(p.qrows, re - rs));

  // largest visible count among the request's rows
  int vm = 0;
  for (int t = rs + tid; t < re; t += 256) vm = max(vm, p.tok_vis[t]);
  for (int o = 32; o > 0; o >>= 1) vm = max(vm, __shfl_xor(vm, o));
  if (lane == 0) s_vmax[wave] = vm;
  __syncthreads();
  int vmax = max(max(s_vmax[0], s_vmax[1]), max(s_vmax[2], s_vmax[3]));
  vmax = min(vmax, p.max_vis);
  const int k0 = blockIdx.x * p.chunk;
  if (k0 >= vmax) return;
  const int kend = min(k0 + p.chunk, vmax);
  const int P = 1 << p.plog2;
  const int lp0 = k0 >> p.plog2;
  for (int i = tid; i <= ((kend - 1) >> p.plog2) - lp0; i += 256)
    pg_lds[i] = phys_page(p.block_table, p.bt_stride, r, lp0 + i, p.num_pages);

  store_rows(min(p.qrows, re - rs));
  for (int t0 = rs;;) {
    const int nr = min(p.qrows, re - t0);
    __syncthreads();

    // Software pipeline: the raw key bytes of round i+1 are in flight while
    // round i is dequantised and multiplied.
    auto mfma_row = [&](int j, const bf16x8 (&bfr)[kIdxKT][4], f32x4 (&acc)[kIdxKT][2]) {
      const __bf16* qrow = &qs[(j * 32) * kQPad];
      (void)qrow;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(&qrow[c * kQPad + kdim<KFMT, false>(kk, g)]);
        const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(&qrow[(16 + c) * kQPad + kdim<KFMT, false>(kk, g)]);
#pragma unroll
        for (int kt = 0; kt < kIdxKT; ++kt) {
          if (kk == 0) {
            acc[kt][0] = mfma16x16x32(a0, bfr[kt][0], f32x4{0.f, 0.f, 0.f, 0.f});
            acc[kt][1] = mfma16x16x32(a1, bfr[kt][0], f32x4{0.f, 0.f, 0.f, 0.f});
          } else {
            acc[kt][0] = mfma16x16x32(a0, bfr[kt][kk], acc[kt][0]);
            acc[kt][1] = mfma16x16x32(a1, bfr[kt][kk], acc[kt][1]);
          }
        }
      }
    };
    // ReLU-weighted head sum: 8 heads in-lane, then a reduce-scatter over the
    // four lane groups leaves lane (g, c) with key c of tile g
    auto epi_row = [&](int j, const f32x4 (&acc)[kIdxKT][2], int s_own, float own_mul) {
      const int vis = s_vis[j];
      const f32x4 w0 = *reinterpret_cast<const f32x4*>(&ws[j * 32 + 4 * g]);
      const f32x4 w1 = *reinterpret_cast<const f32x4*>(&ws[j * 32 + 16 + 4 * g]);
      float v[kIdxKT];
#pragma unroll
      for (int kt = 0; kt < kIdxKT; ++kt) {
        float x = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x += w0[i] * relu(acc[kt][0][i]);
          x += w1[i] * relu(acc[kt][1][i]);
        }
        v[kt] = x;
      }
      const float tot = rows_reduce_scatter4(v);
      if (s_own < kend && s_own < vis)
        p.scores[(int64_t)(t0 + j) * p.ld + s_own] = (own_mul == -__builtin_inff()) ? own_mul : tot * own_mul;
    };
    // FP8 queries: row j's two head tiles against the raw FP8 keys
    auto mfma_row_q8 = [&](int j, const i32x8 (&kb)[kIdxKT], f32x4 (&acc)[kIdxKT][2]) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const uint8_t* qh = qsb + (j * 32 + 16 * hh + c) * kRowB + 32 * g;
        const i32x4 lo = *reinterpret_cast<const i32x4*>(qh), hi = *reinterpret_cast<const i32x4*>(qh + 16);
        const i32x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
        for (int kt = 0; kt < kIdxKT; ++kt) acc[kt][hh] = mfma16x16x128_fp8(a, kb[kt], f32x4{0.f, 0.f, 0.f, 0.f});
      }
    };
    auto do_round = [&](int base, RawKeys<KFMT>& raw, int next) {
      const int s_own = base + wave * (kIdxKT * 16) + lane;  // key this lane stores
      const float own_mul = own_multiplier<KFMT>(raw, g);
      f32x4 acc[kIdxKT][2];
      if constexpr (Q8) {
        i32x8 kb[kIdxKT];
#pragma unroll
        for (int kt = 0; kt < kIdxKT; ++kt) {
          const i32x4 x = raw.v[kt][0], y = raw.v[kt][KFMT == DSA_KEY_FP8 ? 1 : 0];
          kb[kt] = i32x8{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
        }
        if (next < kend) load_round<KFMT>(p, pg_lds, lp0, next, kend, wave, g, c, P, raw);
        for (int j = 0; j < nr; ++j) {
          mfma_row_q8(j, kb, acc);
          epi_row(j, acc, s_own, own_mul);
        }
      } else {
        bf16x8 bfr[kIdxKT][4];
#pragma unroll
        for (int kt = 0; kt < kIdxKT; ++kt) dequant_tile<KFMT>(raw, kt, bfr[kt], raw.sc[kt], g);
        if (next < kend) load_round<KFMT>(p, pg_lds, lp0, next, kend, wave, g, c, P, raw);
        for (int j = 0; j < nr; ++j) {
          mfma_row(j, bfr, acc);
          epi_row(j, acc, s_own, own_mul);
        }
      }
    };

    // Software pipeline: the raw key bytes of round i+1 are in flight while
    // round i is dequantised and multiplied.
    RawKeys<KFMT> raw;
    load_round<KFMT>(p, pg_lds, lp0, k0, kend, wave, g, c, P, raw);
    for (int base = k0; base < kend; base += kIdxRound) do_round(base, raw, base + kIdxRound);

    t0 += p.qrows;
    if (t0 >= re) break;
    __syncthreads();  // every wave is done with this pass's rows
    // later passes (more rows than one pass holds): batches of four loads,
    // which keeps the registers of the round loop free
    const int nr2 = min(p.qrows, re - t0);
    for (int u0 = 0; u0 < kQLoads; u0 += 4) {
      i32x4 b4[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = tid + 256 * (u0 + u);
        const int row = i >> (5 + kPieceLog), head = (i >> kPieceLog) & 31, part = i & ((1 << kPieceLog) - 1);
        if (i < nr2 * kRowPieces) b4[u] = ld16(q_src(t0 + row, head, part));
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = tid + 256 * (u0 + u);
        const int row = i >> (5 + kPieceLog), head = (i >> kPieceLog) & 31, part = i & ((1 << kPieceLog) - 1);
        if (i < nr2 * kRowPieces) *q_dst(row, head, part) = b4[u];
      }
    }
    if (tid < nr2 * 32) ws[tid] = w_of((int64_t)t0 * 32 + tid);
    if (tid < nr2) s_vis[tid] = clamp_vis(p.tok_vis[t0 + tid], p.max_vis);
  }
}

// One query row per request (long-context decode).  The keys stream into a
// private LDS ring per wave by direct HBM -> LDS copies (global_load_lds_
// dwordx4 with the nontemporal hint): a copy moves 1 KiB -- 8 whole FP8 keys
// or 16 whole MXFP4 keys -- so every 128-byte line is fetched by exactly one
// instruction, and the copies are waited for with explicit vmcnt counts,
// so the compiler never drains the stream.  A round is 64 keys per wave
// (four 16-key tiles) plus their 64 side words (FP8 scale / MXFP4 E8M0
// codes); while one round is multiplied the next is in flight.  Inside a
// tile the 16-byte chunk j of key c sits at position c * NC + (j ^ swz(c))
// (NC chunks per key), which makes the fragment reads below conflict-free.
// The row's query fragments stay in registers.
static __device__ __attribute__((aligned(64))) uint8_t g_idx_zero[64] = {0};
__device__ __forceinline__ void idx_dma16(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off nt" : : "v"(src), "s"(lds) : "memory", "m0");
}
__device__ __forceinline__ void idx_dma4(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off nt" : : "v"(src), "s"(lds) : "memory", "m0");
}
template <int N> __device__ __forceinline__ void idx_wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}
__device__ __forceinline__ uint32_t idx_lds_addr(const void* ptr) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)ptr;
}

template <int KFMT> struct KeyStream {
  static constexpr int kKeyBytes = KFMT == DSA_KEY_FP8 ? 128 : 64;  // code bytes per key
  static constexpr int kChunks = kKeyBytes / 16;                     // 16-byte chunks per key
  static constexpr int kCopies = 64 * kKeyBytes / 1024;              // code copies per round
  static constexpr int kSideWords = KFMT == DSA_KEY_NVFP4 ? 2 : 1;   // side dwords per key
  static constexpr int kOps = kCopies + kSideWords;                  // + the side copies
  static constexpr int kRoundBytes = 64 * kKeyBytes + 256 * kSideWords;  // codes, then side words
  static constexpr int kDepth = 2;                                   // rounds per wave ring
  static constexpr int kMaxChunk = KFMT == DSA_KEY_FP8 ? kIndexerRowChunkFp8 : kIndexerRowChunkFp4;
  // swizzle of key c's chunks (c = key within its tile)
  __device__ static int swz(int c) { return KFMT == DSA_KEY_FP8 ? (c >> 1) & 7 : (c >> 2) & 3; }
  // LDS bytes of one workgroup: 4 rings, the chunk's scores, its page ids
  static constexpr size_t kLds = 4 * kDepth * kRoundBytes + kMaxChunk * 4 + (kMaxChunk / 16 + 1) * 4;
};
// FP4 keys fit the default 64 KiB of dynamic LDS; FP8 keys raise the limit
static_assert(KeyStream<DSA_KEY_MXFP4>::kLds <= 65536 && KeyStream<DSA_KEY_NVFP4>::kLds <= 65536, "LDS");
static_assert(KeyStream<DSA_KEY_FP8>::kLds <= 160 * 1024, "LDS");

// QF4 = false: BF16 queries on v_mfma_f32_16x16x32_bf16 over keys dequantised
// exactly to bf16 (any key format).  QF4 = true (MXFP4 keys only): MXFP4
// queries straight into v_mfma_scale_f32_16x16x128_f8f6f4 with both operands
// E2M1 and the E8M0 block scales applied by the instruction (Kimi K3.1 Pro
// page, AMD "native MXFP4 indexer": native FP4 matrix instructions, FP32
// accumulation) -- one instruction per 16 heads x 16 keys x 128 dims, no
// dequantisation.
template <int KFMT, bool QF4>
__global__ __launch_bounds__(256) void indexer_row_kernel(IndexerParams p) {
  static_assert(!QF4 || KFMT == DSA_KEY_MXFP4, "FP4 queries run against MXFP4 keys");
  using KS = KeyStream<KFMT>;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  float* sc_out = reinterpret_cast<float*>(lds + 4 * KS::kDepth * KS::kRoundBytes);  // [chunk]
  int* pg_lds = reinterpret_cast<int*>(sc_out + KS::kMaxChunk);                       // [chunk/16 + 1]
  const int r = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c = lane & 15;
  const int k0 = blockIdx.x * p.chunk;
  const int kcap = min(k0 + p.chunk, p.max_vis);  // chunk end before the row's visible count is known
  const int P = 1 << p.plog2;
  const int lp0 = k0 >> p.plog2;
  // Prologue, shortest dependency chain first: the chunk's page ids and the
  // row index do not depend on each other; the first copies go out as soon
  // as the page ids are in LDS, before the row's visible count and query
  // arrive (keys past the visible count are read but never stored).
  for (int i = tid; i <= ((kcap - 1) >> p.plog2) - lp0; i += 256)
    pg_lds[i] = phys_page(p.block_table, p.bt_stride, r, lp0 + i, p.num_pages);
  // (loaded values are uniform; saying so keeps the round bookkeeping scalar)
  const int t_first = __builtin_amdgcn_readfirstlane(p.req_row_start[r]);
  const int t_end = __builtin_amdgcn_readfirstlane(p.req_row_start[r + 1]);
  __syncthreads();

  uint8_t* ring = lds + wave * KS::kDepth * KS::kRoundBytes;
  const uint32_t ring_l = idx_lds_addr(ring);
  // Copies of round `it` into ring slot it % kDepth.  Keys at or past `kc`
  // are clamped onto key kc - 1, so every round issues the same copies.
  // Side words: the FP8 scale or MXFP4 E8M0 word of the lane's key at word
  // `lane`; NVFP4 scale bytes 0..3 at word `lane`, 4..7 at word 64 + lane.
  auto issue = [&](int it, int kc) {
    const int kb = k0 + it * kIdxRound + wave * 64;  // first key of the wave's share
    const int own = min(kb + lane, kc - 1);           // this lane's key (clamped)
    const int pg_own = pg_lds[(own >> p.plog2) - lp0];
    const uint32_t slot_l = ring_l + (it % KS::kDepth) * KS::kRoundBytes;
#pragma unroll
    for (int d = 0; d < KS::kCopies; ++d) {
      // copy d: tile kt, keys cb .. cb + 1024 / kKeyBytes - 1 of the tile
      constexpr int kPerCopy = 1024 / KS::kKeyBytes;
      const int kt = d * kPerCopy / 16, cb = d * kPerCopy % 16;
      const int cc = cb + lane / KS::kChunks;                 // key within the tile
      const int j = (lane % KS::kChunks) ^ KS::swz(cc);      // its chunk this lane moves
      const int pg = __builtin_amdgcn_readlane(pg_own, kt * 16);  // the tile lies in one page
      const int key = min(kb + kt * 16 + cc, kc - 1);
      const uint8_t* src = pg >= 0 ? p.keys + (int64_t)pg * p.page_bytes + (key & (P - 1)) * KS::kKeyBytes + j * 16
                                   : g_idx_zero;
      idx_dma16(src, slot_l + d * 1024);
    }
    constexpr int kSideBytes = 4 * KS::kSideWords;
#pragma unroll
    for (int w = 0; w < KS::kSideWords; ++w) {
      const uint8_t* sw = pg_own >= 0 ? p.keys + (int64_t)pg_own * p.page_bytes + P * KS::kKeyBytes +
                                            (own & (P - 1)) * kSideBytes + 4 * w
                                      : g_idx_zero;
      idx_dma4(sw, slot_l + 64 * KS::kKeyBytes + 256 * w);
    }
  };
  // rounds the chunk can have before its visible count is known
  const int nround_cap = (kcap - k0 + kIdxRound - 1) / kIdxRound;
  const int nfirst = min(KS::kDepth, nround_cap);

  // One row per request is the intended shape; further rows of the request
  // (more than the host bound promised) are scored the same way in turn.
  for (int t = t_first; t < t_end; ++t) {
    for (int d = 0; d < nfirst; ++d) issue(d, kcap);
    int issued = nfirst;  // rounds issued so far (round i uses ring slot i % kDepth)

    // the row's visible count, query fragments and head weights
    const int vis = __builtin_amdgcn_readfirstlane(clamp_vis(p.tok_vis[t], p.max_vis));
    bf16x8 qa[2][4];
    i32x4 q4[2];      // QF4: E2M1 codes of head 16hh + c, dims 32g .. 32g+31
    uint32_t qe[2];   // QF4: their E8M0 scale
    if (QF4) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        q4[hh] = ld16(p.q8 + ((int64_t)t * 32 + 16 * hh + c) * 64 + 16 * g);
        qe[hh] = p.q_e8m0[((int64_t)t * 32 + 16 * hh + c) * 4 + g];
      }
    } else {
      const __bf16* qrow = p.q + (int64_t)t * 32 * 128;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          qa[hh][kk] = __builtin_bit_cast(bf16x8, ld16(qrow + (16 * hh + c) * 128 + kdim<KFMT, true>(kk, g)));
    }
    const f32x4 w0 = *reinterpret_cast<const f32x4*>(p.w + (int64_t)t * 32 + 4 * g);
    const f32x4 w1 = *reinterpret_cast<const f32x4*>(p.w + (int64_t)t * 32 + 16 + 4 * g);
    // These loads must be complete, and known to the compiler to be, before the
    // loop: one still pending there would make the compiler wait for every copy
    // in flight on every round.  (This wait also covers the first copies.)
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    if (k0 >= vis) continue;              // nothing in flight (vis is uniform)
    const int kend = min(kcap, vis);
    const int nround = (kend - k0 + kIdxRound - 1) / kIdxRound;

    static_assert(KS::kDepth >= 2 && KS::kDepth <= 4, "wait counts for 1 .. 3 rounds behind");
    for (int it = 0; it < nround; ++it) {
      // rounds it+1 .. issued-1 are the copies issued after round it's
      switch (issued - 1 - it) {
        case 0: idx_wait_vmcnt<0>(); break;
        case 1: idx_wait_vmcnt<KS::kOps>(); break;
        case 2: idx_wait_vmcnt<2 * KS::kOps>(); break;
        default: idx_wait_vmcnt<3 * KS::kOps>(); break;
      }
      const uint8_t* rd = ring + (it % KS::kDepth) * KS::kRoundBytes;
      const uint32_t* side = reinterpret_cast<const uint32_t*>(rd + 64 * KS::kKeyBytes);
      float v[kIdxKT];
#pragma unroll
      for (int kt = 0; kt < kIdxKT; ++kt) {
        const uint8_t* tile = rd + kt * 16 * KS::kKeyBytes + c * KS::kKeyBytes;
        bf16x8 b[4];
        f32x4 a0, a1;
        if (QF4) {
          // key c's codes of dims 32g .. 32g+31 and their E8M0 scale g
          const i32x4 x = *reinterpret_cast<const i32x4*>(tile + (g ^ KS::swz(c)) * 16);
          const uint32_t ke = (side[kt * 16 + c] >> (8 * g)) & 0xFFu;
          a0 = mfma16x16x128_fp4(q4[0], qe[0], x, ke, f32x4{0.f, 0.f, 0.f, 0.f});
          a1 = mfma16x16x128_fp4(q4[1], qe[1], x, ke, f32x4{0.f, 0.f, 0.f, 0.f});
        } else if (KFMT == DSA_KEY_FP8) {
          const i32x4 x = *reinterpret_cast<const i32x4*>(tile + (g ^ KS::swz(c)) * 16);
          const i32x4 y = *reinterpret_cast<const i32x4*>(tile + ((4 + g) ^ KS::swz(c)) * 16);
          b[0] = e4m3x8_to_bf16x8(x[0], x[1]);
          b[1] = e4m3x8_to_bf16x8(x[2], x[3]);
          b[2] = e4m3x8_to_bf16x8(y[0], y[1]);
          b[3] = e4m3x8_to_bf16x8(y[2], y[3]);
        } else if (KFMT == DSA_KEY_MXFP4) {
          const i32x4 x = *reinterpret_cast<const i32x4*>(tile + (g ^ KS::swz(c)) * 16);
          const float sc = e8m0_to_f32((side[kt * 16 + c] >> (8 * g)) & 0xFFu);
          b[0] = e2m1x8_to_bf16x8(x[0], sc);
          b[1] = e2m1x8_to_bf16x8(x[1], sc);
          b[2] = e2m1x8_to_bf16x8(x[2], sc);
          b[3] = e2m1x8_to_bf16x8(x[3], sc);
        } else {
          // NVFP4: dims 32g .. 32g+31 are blocks 2g, 2g+1: scale bytes 2g, 2g+1
          // of the key, i.e. half (g & 1) of side word (g >> 1)
          const i32x4 x = *reinterpret_cast<const i32x4*>(tile + (g ^ KS::swz(c)) * 16);
          const uint32_t sw = side[(g >> 1) * 64 + kt * 16 + c] >> (16 * (g & 1));
          const float s0 = e4m3_to_f32(sw & 0xFFu), s1 = e4m3_to_f32((sw >> 8) & 0xFFu);
          b[0] = e2m1x8_times(x[0], s0);
          b[1] = e2m1x8_times(x[1], s0);
          b[2] = e2m1x8_times(x[2], s1);
          b[3] = e2m1x8_times(x[3], s1);
        }
        if (!QF4) {
          a0 = mfma16x16x32(qa[0][0], b[0], f32x4{0.f, 0.f, 0.f, 0.f});
          a1 = mfma16x16x32(qa[1][0], b[0], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
          for (int kk = 1; kk < 4; ++kk) {
            a0 = mfma16x16x32(qa[0][kk], b[kk], a0);
            a1 = mfma16x16x32(qa[1][kk], b[kk], a1);
          }
        }
        float x = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x += w0[i] * relu(a0[i]);
          x += w1[i] * relu(a1[i]);
        }
        v[kt] = x;
      }
      // lane stores key k0 + it * 256 + wave * 64 + lane: its multiplier is the
      // FP8 scale (1 for MXFP4 / NVFP4) on a present page, -inf otherwise
      const int s_own = k0 + it * kIdxRound + wave * 64 + lane;
      const int pg_own = pg_lds[(min(s_own, kend - 1) >> p.plog2) - lp0];
      const float mul = pg_own < 0 ? -__builtin_inff() : (KFMT == DSA_KEY_FP8 ? __uint_as_float(side[lane]) : 1.f);
      const float tot = rows_reduce_scatter4(v);
      if (s_own < kend) sc_out[s_own - k0] = mul == -__builtin_inff() ? mul : tot * mul;
      // the slot is read; refill it with the next round (if the chunk has one)
      if (issued < nround) {
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        issue(issued, kend);
        ++issued;
      }
    }
    idx_wait_vmcnt<0>();  // no copy may land after the workgroup's LDS is released
    __syncthreads();
    float* out = p.scores + (int64_t)t * p.ld;
    // Nontemporal stores: the scores are read once, by the top-k, and a store
    // that allocates in the caches evicts (and writes back) whatever dirty
    // lines they hold while the key stream runs (measured: 241 -> 213 us on
    // the 64-request 256K MXFP4 batch, 110 -> 101 us at 1M; the top-k then
    // reads the scores from HBM, 4-8 us more)
    for (int i = tid; i < kend - k0; i += 256) __builtin_nontemporal_store(sc_out[i], out + k0 + i);
    if (t + 1 < t_end) __syncthreads();  // the next row rewrites the rings and sc_out
  }
}

// Shared-prefix plan.  Groups are cut into sub-groups of at most
// kPrefixSubRows rows (serially, one thread: there are few groups), padded
// with empty sub-groups up to the bound the host sized the grid for; then the
// visible counts of the prefix and suffix passes, and every sub-group's copy
// of its group's prefix pages (read from the block-table row of one of its
// requests; a bad request id gives absent pages).
__global__ void prefix_groups_kernel(const int32_t* __restrict__ grs, int G, int T, int ns_max,
                                     int32_t* __restrict__ sub_start, int32_t* __restrict__ sub_src) {
  if (blockIdx.x != 0 || threadIdx.x != 0) return;
  int ns = 0;
  for (int g = 0; g < G && ns < ns_max; ++g) {
    const int s = min(max(grs[g], 0), T), e = min(max(grs[g + 1], s), T);
    for (int x = s; x < e && ns < ns_max; x += kPrefixSubRows) {
      sub_start[ns] = x;
      sub_src[ns] = g;
      ++ns;
    }
  }
  for (; ns < ns_max; ++ns) {
    sub_start[ns] = T;
    sub_src[ns] = -1;
  }
  sub_start[ns_max] = T;
}

__global__ void prefix_prep_kernel(const int32_t* __restrict__ tok_vis, int T, int max_vis, int L,
                                   const int32_t* __restrict__ bt, int bt_stride, int R,
                                   const int32_t* __restrict__ first_req, const int32_t* __restrict__ sub_src,
                                   int ns, int npfx, int32_t* __restrict__ vis1, int32_t* __restrict__ vis2,
                                   int32_t* __restrict__ ptab) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < T) {
    const int v = min(max(tok_vis[i], 0), max_vis);
    vis1[i] = min(v, L);
    vis2[i] = max(v - L, 0);
  }
  if (i < ns * npfx) {
    const int q = i / npfx, j = i - q * npfx;
    const int g = sub_src[q];
    const int r = g >= 0 ? first_req[g] : -1;
    ptab[i] = (r >= 0 && r < R) ? bt[(int64_t)r * bt_stride + j] : -1;
  }
}

dsa_status launch_prefix_prep(const int32_t* tok_vis, int T, int max_vis, int L, const int32_t* bt, int bt_stride,
                              int R, const int32_t* grs, const int32_t* first_req, int G, int ns_max, int npfx,
                              int32_t* sub_start, int32_t* sub_src, int32_t* vis1, int32_t* vis2, int32_t* ptab,
                              hipStream_t stream) {
  hipLaunchKernelGGL(prefix_groups_kernel, dim3(1), dim3(64), 0, stream, grs, G, T, ns_max, sub_start, sub_src);
  const int n = max(T, ns_max * npfx);
  hipLaunchKernelGGL(prefix_prep_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, tok_vis, T, max_vis, L, bt,
                     bt_stride, R, first_req, sub_src, ns_max, npfx, vis1, vis2, ptab);
  return hipGetLastError() == hipSuccess ? DSA_OK : DSA_ERR_HIP;
}

dsa_status launch_indexer_bf16(const IndexerParams& p, hipStream_t stream) {
  dim3 grid((p.max_vis + p.chunk - 1) / p.chunk, p.R);
  const size_t lds = (size_t)p.qrows * 32 * (kQPad * sizeof(__bf16) + sizeof(float));
  if (p.q_e8m0) {
    // MXFP4 queries: the streaming kernel on the FP4 matrix instruction, every
    // row of a request in turn
    hipLaunchKernelGGL((indexer_row_kernel<DSA_KEY_MXFP4, true>), grid, dim3(256), KeyStream<DSA_KEY_MXFP4>::kLds,
                       stream, p);
  } else if (p.q8) {
    // FP8 queries of few-row requests (decode): FP8 keys only (checked by the caller)
    const size_t lds8 = (size_t)p.qrows * 32 * (kQ8Pad + sizeof(float));
    hipLaunchKernelGGL((indexer_bf16_kernel<DSA_KEY_FP8, true>), grid, dim3(256), lds8, stream, p);
  } else if (p.max_rows_per_req == 1) {
    if (p.key_fmt == DSA_KEY_FP8) {
      // above the default 64 KiB of dynamic LDS (idempotent, host-side)
      if (hipFuncSetAttribute(reinterpret_cast<const void*>(indexer_row_kernel<DSA_KEY_FP8, false>),
                              hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)KeyStream<DSA_KEY_FP8>::kLds) != hipSuccess)
        return DSA_ERR_HIP;
      hipLaunchKernelGGL((indexer_row_kernel<DSA_KEY_FP8, false>), grid, dim3(256), KeyStream<DSA_KEY_FP8>::kLds,
                         stream, p);
    } else if (p.key_fmt == DSA_KEY_MXFP4) {
      hipLaunchKernelGGL((indexer_row_kernel<DSA_KEY_MXFP4, false>), grid, dim3(256), KeyStream<DSA_KEY_MXFP4>::kLds,
                         stream, p);
    } else {
      hipLaunchKernelGGL((indexer_row_kernel<DSA_KEY_NVFP4, false>), grid, dim3(256), KeyStream<DSA_KEY_NVFP4>::kLds,
                         stream, p);
    }
  } else if (p.key_fmt == DSA_KEY_FP8) {
    hipLaunchKernelGGL((indexer_bf16_kernel<DSA_KEY_FP8, false>), grid, dim3(256), lds, stream, p);
  } else if (p.key_fmt == DSA_KEY_MXFP4) {
    hipLaunchKernelGGL((indexer_bf16_kernel<DSA_KEY_MXFP4, false>), grid, dim3(256), lds, stream, p);
  } else {
    hipLaunchKernelGGL((indexer_bf16_kernel<DSA_KEY_NVFP4, false>), grid, dim3(256), lds, stream, p);
  }
  return hipGetLastError() == hipSuccess ? DSA_OK : DSA_ERR_HIP;
}

DSA_DEBUG_TAKE(indexer)

}  // namespace dsa
