// Lightning-indexer scores on gfx950 MFMA.
//
//   I(t, s) = index_scale * sum_j w[t, j] * max(0, q_idx[t, j, :] . k[slot(b, s), :])
//
// (scoring stage of tokenspeed PR 627 "Add gluon kernel for DSA"; keys are the paged
// index_k_cache of the decode top-k wrapper in that PR's review, bf16, or fp8 e4m3 with an
// fp32 per-token scale.)
//
// A CU sustains only ~25 GB/s of HBM reads, so the stream is spread as one 8-wave workgroup
// per CU and the row's query heads are fetched once per workgroup. A wave owns tiles of 64
// consecutive candidate positions of one query row. The row's query
// heads are the MFMA A operand (M = 16 heads per tile; staged once per workgroup through LDS,
// then held in registers), the 64 keys are four B operands of 16 keys each (K = 32 dims per
// MFMA), loaded straight from HBM into registers: lane l reads 16 (bf16) or 8 (fp8)
// contiguous bytes of key l%16, so each load instruction covers 64 contiguous bytes of 16 rows
// and a tile is one contiguous 16 KiB (bf16, page 64) or 8 KiB (fp8) burst. The query heads
// are requested first (every MFMA waits on them), the first tile's keys right after, and
// every later tile is prefetched one step ahead. The epilogue applies ReLU and the
// head weights in fp32 on the accumulators, reduce-scatters over the four lane groups with
// three lane swaps so lane l ends up with candidate s0 + l, and stores one coalesced 256-byte
// row segment. Optionally the same pass counts a 4096-bin histogram of the top 12 bits of
// the order-preserving key of each score (first radix digit of the top-k select).
#include "common.hpp"
#include "kernels.hpp"

namespace dsa {

// Keys of one 64-candidate tile as four B operands (16 keys each); fp8 keys are widened to
// bf16 (exact) and their per-token scale kept for the epilogue.
template <int DI, bool FP8>
struct KeyTile {
  static constexpr int KB = DI / 32;
  u32x4_t b[4][KB];
  float sc[4];

  // Addressing of the tile's four 16-key sub-tiles for this lane's key c, in two halves so
  // that the page-table reads of two tiles go out together and well before their key loads:
  // table() issues the reads (raw entries + in-page offsets; packed caches: the positions),
  // finish() turns them into clamped slots.
  struct Addr {
    int pg[4];
    int off[4];
  };
  // Branch-free (a merge after a conditional read would force a wait right after it): a
  // paged cache reads its block-table entry, a packed cache reads req_base[b] through the same
  // load.
  __device__ __forceinline__ static void table(const ScoreArgs& a, int b_req, int s0, int n, int c,
                                               Addr& ad) {
    const Paging& p = a.pg;
    const bool paged = p.bt != nullptr;
    const int32_t* tb = paged ? p.bt : p.req_base;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int pos = min(s0 + 16 * st + c, n - 1);
      const int q = p.page_shift >= 0 ? (pos >> p.page_shift) : pos / p.page;
      const int lp = min(max(q, 0), max((int)p.bt_stride - 1, 0));
      ad.off[st] = paged ? pos - q * p.page : pos;
      const int64_t at = paged ? (int64_t)b_req * p.bt_stride + lp : (int64_t)b_req;
      ad.pg[st] = tb[at];
    }
  }
  __device__ __forceinline__ static void finish(const ScoreArgs& a, const Addr& ad, int64_t* sl) {
    const Paging& p = a.pg;
    const bool paged = p.bt != nullptr;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int64_t in_page = (int64_t)min(max(ad.pg[st], 0), p.n_pages - 1) * p.page + ad.off[st];
      const int64_t v = (int64_t)ad.pg[st] + ad.off[st];
      const int64_t packed = v < 0 ? 0 : (v >= p.n_slots ? p.n_slots - 1 : v);
      sl[st] = paged ? in_page : packed;
    }
  }

  __device__ __forceinline__ void load(const ScoreArgs& a, const int64_t* sl, int g) {
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int64_t slot = sl[st];
      if constexpr (!FP8) {
        const uint16_t* kp = reinterpret_cast<const uint16_t*>(a.keys) + slot * DI + 8 * g;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) b[st][kb] = *reinterpret_cast<const u32x4_t*>(kp + 32 * kb);
        sc[st] = 1.0f;
      } else {
        const uint8_t* kp = reinterpret_cast<const uint8_t*>(a.keys) + slot * DI + 8 * g;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const u32x2_t raw = *reinterpret_cast<const u32x2_t*>(kp + 32 * kb);
          b[st][kb] = u32x4_t{raw[0], raw[1], 0u, 0u};   // widened after the loads land
        }
        sc[st] = a.key_scale[slot];
      }
    }
  }

  __device__ __forceinline__ void widen() {
    if constexpr (FP8) {
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) b[st][kb] = fp8x8_to_bf16x8(u32x2_t{b[st][kb][0], b[st][kb][1]});
    }
  }
};

constexpr int kScoreWaves = 8;   // one 512-thread workgroup per CU: the query heads load once per CU
constexpr int kScoreThreads = 64 * kScoreWaves;

template <int DI, int MT, bool FP8, bool HIST>
__global__ __launch_bounds__(kScoreThreads) void k_index_scores(ScoreArgs a) {
  constexpr int KB = DI / 32;
  // the row's query heads in LDS, one head per QS bytes: the 16 bytes of padding put the 16
  // heads that one A-operand read touches in distinct banks
  constexpr int QS = DI * 2 + 16;
  __shared__ __align__(16) uint8_t s_q[64 * QS];
  __shared__ float s_w[16 * MT];
  __shared__ uint32_t s_hist[HIST ? kHistBins : 1];

  const int t = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4;       // lane group 0..3
  const int c = lane & 15;       // column within a 16-wide tile
  const int stride = gridDim.x * kScoreWaves;
  int tile = blockIdx.x * kScoreWaves + wave;

  // 1. page-table entries of this wave's first two tiles, 2. the row's query heads and head
  // weights (staged once per workgroup in LDS, zero-padded to 16 * MT heads), 3. the first
  // tile's 16 key loads back to back. Loads complete in issue order, so each wait below only
  // covers what it needs. The table reads do not wait for the row's request and length: they
  // go out for request t (a decode row is its own request) and the longest row, both kept
  // inside the table, and are re-issued only if the row belongs to another request.
  using Tile = KeyTile<DI, FP8>;
  typename Tile::Addr ad_cur, ad_nxt;
  const int b_spec = min(t, a.n_req - 1);
  const int ntiles_max = (a.n_max + 63) >> 6;
  if (tile < ntiles_max) Tile::table(a, b_spec, tile << 6, a.n_max, c, ad_cur);
  if (tile + stride < ntiles_max) Tile::table(a, b_spec, (tile + stride) << 6, a.n_max, c, ad_nxt);
  const int b = min(max(a.row_req ? a.row_req[t] : t, 0), a.n_req - 1);
  int n = a.row_len[t];
  n = min(max(n, 0), a.n_max);
  const int ntiles = (n + 63) >> 6;
  if (b != b_spec) {   // uniform: the whole workgroup serves row t
    if (tile < ntiles) Tile::table(a, b, tile << 6, n, c, ad_cur);
    if (tile + stride < ntiles) Tile::table(a, b, (tile + stride) << 6, n, c, ad_nxt);
  }
  constexpr int QPT = (16 * MT * DI * 2 + kScoreThreads * 16 - 1) / (kScoreThreads * 16);
  u32x4_t qv[QPT];
  {
    const uint8_t* qrow = reinterpret_cast<const uint8_t*>(a.q_idx + (int64_t)t * a.ld_q);
    const int qbytes = a.Hi * DI * 2;
#pragma unroll
    for (int i = 0; i < QPT; ++i) {
      const int o = (threadIdx.x + i * kScoreThreads) * 16;
      qv[i] = o < qbytes ? *reinterpret_cast<const u32x4_t*>(qrow + o) : u32x4_t{0u, 0u, 0u, 0u};
    }
  }
  const float wraw = threadIdx.x < a.Hi ? a.w[(int64_t)t * a.ld_w + threadIdx.x] : 0.0f;
  // q and w arrive with the table entries; staging them first keeps the key loads below clear
  // of any wait
#pragma unroll
  for (int i = 0; i < QPT; ++i) {
    const int o = (threadIdx.x + i * kScoreThreads) * 16;
    if (o < 16 * MT * DI * 2) *reinterpret_cast<u32x4_t*>(s_q + (o / (DI * 2)) * QS + o % (DI * 2)) = qv[i];
  }
  if (threadIdx.x < 16 * MT) s_w[threadIdx.x] = wraw * a.index_scale;
  if constexpr (HIST)
    for (int i = threadIdx.x; i < kHistBins; i += kScoreThreads) s_hist[i] = 0;
  Tile cur;
  if (tile < ntiles) {
    int64_t sl[4];
    Tile::finish(a, ad_cur, sl);
    cur.load(a, sl, g);
  }
  lds_barrier();   // not __syncthreads(): the first tile's key loads stay in flight
  // A operands: qa[mt][kb] = q_idx[t, 16 mt + c, 32 kb + 8 g .. +7]; weights of the
  // accumulator rows this lane holds (row r of head tile mt is head 16 mt + 4 g + r)
  u32x4_t qa[MT][KB];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
      qa[mt][kb] = *reinterpret_cast<const u32x4_t*>(s_q + (16 * mt + c) * QS + (32 * kb + 8 * g) * 2);
  float wv[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) wv[mt][r] = s_w[16 * mt + 4 * g + r];

  while (tile < ntiles) {
    const int s0 = tile << 6;
    const int next = tile + stride;
    Tile nxt;
    if (next < ntiles) {                                       // prefetch the next tile
      int64_t sl[4];
      Tile::finish(a, ad_nxt, sl);
      nxt.load(a, sl, g);
    }
    if (next + stride < ntiles) Tile::table(a, b, (next + stride) << 6, n, c, ad_nxt);
    cur.widen();
    float part[4];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      f32x4_t acc[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt] = mfma_bf16_16x16x32(qa[mt][kb], cur.b[st][kb], acc[mt]);
      float p = 0.f;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float x = acc[mt][r];
          if constexpr (FP8) x *= cur.sc[st];
          p = fmaf(wv[mt][r], relu_f32(x), p);
        }
      part[st] = p;
    }
    // reduce-scatter over the 4 lane groups: group g keeps the full sum of sub-tile st = g
    const float total = reduce_scatter_rows4(part[0], part[1], part[2], part[3]);

    const int s = s0 + lane;
    if (s < n) {
      a.logits[(int64_t)t * a.ld_logits + s] = total;
      if constexpr (HIST) atomicAdd(&s_hist[float_key(total) >> (32 - kHistBits)], 1u);
    }
    cur = nxt;
    tile = next;
  }

  if constexpr (HIST) {
    lds_barrier();
    if (ntiles > 0) {
      uint32_t* gh = a.hist + ((int64_t)t * kHistSlices + (blockIdx.x % kHistSlices)) * kHistBins;
      for (int i = threadIdx.x; i < kHistBins; i += kScoreThreads) {
        const uint32_t v = s_hist[i];
        if (v) atomicAdd(gh + i, v);
      }
    }
  }
}

template <int DI, int MT, bool FP8, bool HIST>
static hipError_t launch_t(const ScoreArgs& a, int T, hipStream_t st) {
  const int ntiles = (a.n_max + 63) / 64;
  int gx = (ntiles + kScoreWaves - 1) / kScoreWaves;
  // about one workgroup per CU in total: longer rows loop (with prefetch) inside the waves
  const int cap = max(1, 256 / T);
  gx = max(1, min(gx, cap));
  launch_kernel(k_index_scores<DI, MT, FP8, HIST>, dim3(gx, T), dim3(kScoreThreads), st, a);
  return hipGetLastError();
}

template <int DI, bool FP8, bool HIST>
static hipError_t launch_mt(const ScoreArgs& a, int T, hipStream_t st) {
  if (a.Hi <= 16) return launch_t<DI, 1, FP8, HIST>(a, T, st);
  if (a.Hi <= 32) return launch_t<DI, 2, FP8, HIST>(a, T, st);
  return launch_t<DI, 4, FP8, HIST>(a, T, st);
}

template <bool FP8, bool HIST>
static hipError_t launch_di(const ScoreArgs& a, int di, int T, hipStream_t st) {
  if (di == 64) return launch_mt<64, FP8, HIST>(a, T, st);
  return launch_mt<128, FP8, HIST>(a, T, st);
}

hipError_t launch_index_scores(const ScoreArgs& a, int di, bool fp8, bool hist, int T,
                               hipStream_t st) {
  if (T <= 0 || a.n_max <= 0) return hipSuccess;
  if (fp8) return hist ? launch_di<true, true>(a, di, T, st) : launch_di<true, false>(a, di, T, st);
  return hist ? launch_di<false, true>(a, di, T, st) : launch_di<false, false>(a, di, T, st);
}

}  // namespace dsa
