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
// are requested first (every MFMA waits on them), the first tile's keys right after. Later
// tiles stream through a ring of the four sub-tile buffers (each refilled with the next tile's
// sub-tile as soon as it is computed), their page-table entries read a tile earlier, so a
// wave always has 16 KiB of keys in flight and never drains between tiles. The epilogue applies ReLU and the
// head weights in fp32 on the accumulators, reduce-scatters over the four lane groups with
// three lane swaps so lane l ends up with candidate s0 + l, and stores one coalesced 256-byte
// row segment. Optionally the same pass counts a 4096-bin histogram of the top 12 bits of
// the order-preserving key of each score (first radix digit of the top-k select).
#include "common.hpp"
#include "kernels.hpp"

namespace dsa {

// Page-table addressing of a 64-candidate tile (this lane's key c of each 16-key sub-tile),
// and the keys of one 16-key sub-tile as B operands (fp8 keys stay raw until use).
template <int DI, bool FP8>
struct KeyTile {
  static constexpr int KB = DI / 32;

  // Addressing of the tile's four 16-key sub-tiles for this lane's key c, in two halves so
  // that the page-table reads go out well before their key loads: table() issues the reads
  // (raw entries + in-page offsets; packed caches: the positions), finish() turns them into
  // clamped slots.
  struct Addr {
    int pg[4];
    int off[4];
  };
  // Branch-free (a merge after a conditional read would force a wait right after it): a
  // paged cache reads its block-table entry, a packed cache reads req_base[b] through the same
  // load. Positions past the row read its last position's entry.
  __device__ __forceinline__ static void table(const ScoreArgs& a, int b_req, int s0, int n, int c,
                                               Addr& ad) {
    const Paging& p = a.pg;
    const bool paged = p.bt != nullptr;
    const int32_t* tb = paged ? p.bt : p.req_base;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int pos = max(min(s0 + 16 * st + c, n - 1), 0);
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

  // One 16-key sub-tile: bf16 keys as B operands, or the raw fp8 bytes and the key's scale.
  struct Sub {
    u32x4_t b[FP8 ? 1 : KB];
    u32x2_t r[FP8 ? KB : 1];
    float sc;
  };
  __device__ __forceinline__ static void load(const ScoreArgs& a, int64_t slot, int g, Sub& k) {
    if constexpr (!FP8) {
      const uint16_t* kp = reinterpret_cast<const uint16_t*>(a.keys) + slot * DI + 8 * g;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        k.b[kb] = *reinterpret_cast<const u32x4_t*>(kp + 32 * kb);
    } else {
      const uint8_t* kp = reinterpret_cast<const uint8_t*>(a.keys) + slot * DI + 8 * g;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        k.r[kb] = *reinterpret_cast<const u32x2_t*>(kp + 32 * kb);
      k.sc = a.key_scale[slot];
    }
  }
  // the B operand of k-step kb: fp8 bytes widened to bf16 by gfx950's scaled conversion at
  // scale 1 (one instruction per two keys; exact, an e4m3 value fits bf16)
  __device__ __forceinline__ static u32x4_t operand(const Sub& k, int kb) {
    if constexpr (FP8) {
      const u32x2_t w = k.r[kb];
      return u32x4_t{fp8x2_to_bf16x2_pow2<false>(w[0], 1.0f), fp8x2_to_bf16x2_pow2<true>(w[0], 1.0f),
                     fp8x2_to_bf16x2_pow2<false>(w[1], 1.0f), fp8x2_to_bf16x2_pow2<true>(w[1], 1.0f)};
    } else {
      return k.b[kb];
    }
  }
};

constexpr int kScoreWaves = 8;   // one 512-thread workgroup per CU: the query heads load once per CU
constexpr int kScoreThreads = 64 * kScoreWaves;

// WHOLE: every 64-candidate tile lies inside one page (a page size that is a multiple of 64,
// or a packed cache), so a tile's slots are one base slot plus the in-tile position.
template <int DI, int MT, bool FP8, bool HIST, bool WHOLE>
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

  // 1. page-table entries of this wave's first tiles, 2. the row's query heads and head
  // weights (staged once per workgroup in LDS, zero-padded to 16 * MT heads), 3. the first
  // tile's 16 key loads back to back. Loads complete in issue order, so each wait below only
  // covers what it needs. The table reads do not wait for the row's request and length: they
  // go out for request t (a decode row is its own request) and the longest row, both kept
  // inside the table, and are re-issued only if the row belongs to another request.
  using Tile = KeyTile<DI, FP8>;
  typename Tile::Addr ad0, ad;    // the first tile's table entries; then those of the next tile
  const int tile0 = tile;
  const int b_spec = min(t, a.n_req - 1);
  const int ntiles_max = (a.n_max + 63) >> 6;
  // WHOLE: lane j holds the table entry (packed cache: the request's base slot) of the wave's
  // tile tile0 + (k0 + j) stride, for the 64 steps from k0; a tile's entry is read from its lane
  const Paging& pgs = a.pg;
  auto entries = [&](int b_req, int k0, int n_c) {
    const int tl = min(tile0 + (k0 + lane) * stride, max((n_c + 63) >> 6, 1) - 1);
    if (pgs.bt) {
      const int s0 = tl << 6;
      const int q = pgs.page_shift >= 0 ? (s0 >> pgs.page_shift) : s0 / pgs.page;
      const int lp = min(max(q, 0), max((int)pgs.bt_stride - 1, 0));
      return pgs.bt[(int64_t)b_req * pgs.bt_stride + lp];
    }
    return pgs.req_base[b_req];
  };
  int ent = 0;
  if constexpr (WHOLE) {
    ent = entries(b_spec, 0, a.n_max);
  } else {
    if (tile < ntiles_max) Tile::table(a, b_spec, tile << 6, a.n_max, c, ad0);
    if (tile + stride < ntiles_max) Tile::table(a, b_spec, (tile + stride) << 6, a.n_max, c, ad);
  }
  const int b = min(max(a.row_req ? a.row_req[t] : t, 0), a.n_req - 1);
  int n = a.row_len[t];
  n = min(max(n, 0), a.n_max);
  const int ntiles = (n + 63) >> 6;
  if (b != b_spec) {   // uniform: the whole workgroup serves row t
    if constexpr (WHOLE) {
      ent = entries(b, 0, n);
    } else {
      if (tile < ntiles) Tile::table(a, b, tile << 6, n, c, ad0);
      if (tile + stride < ntiles) Tile::table(a, b, (tile + stride) << 6, n, c, ad);
    }
  }
  // WHOLE: the slots of tile tl for this lane's key c of each sub-tile, from the tile's entry
  auto whole_slots = [&](int tl, int e, int64_t* sl) {
    const int s0 = tl << 6;
    if (pgs.bt) {
      const int in_page = pgs.page_shift >= 0 ? (s0 & (pgs.page - 1)) : s0 % pgs.page;
      const int64_t base = (int64_t)min(max(e, 0), pgs.n_pages - 1) * pgs.page + in_page;
#pragma unroll
      for (int st = 0; st < 4; ++st) sl[st] = base + 16 * st + c;
    } else {
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const int64_t v = (int64_t)e + s0 + 16 * st + c;
        sl[st] = v < 0 ? 0 : (v >= pgs.n_slots ? pgs.n_slots - 1 : v);
      }
    }
  };
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
  // The keys stream through a ring of the four 16-key sub-tile buffers: as soon as sub-tile st
  // of a tile is computed, its registers take sub-tile st of the wave's next tile, so a tile
  // of keys (16 KiB bf16) is in flight at every wait, with no drain between tiles (the copy of
  // a whole prefetched tile into the working one waited for all of its loads: 10% slower at 1M
  // candidates).
  typename Tile::Sub ring[4];
  if (tile < ntiles) {
    int64_t sl[4];
    if constexpr (WHOLE) whole_slots(tile, __builtin_amdgcn_readfirstlane(ent), sl);
    else Tile::finish(a, ad0, sl);
#pragma unroll
    for (int st = 0; st < 4; ++st) Tile::load(a, sl[st], g, ring[st]);
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

  // One 16-key sub-tile: this lane's share of the weighted ReLU head sum of its key c.
  auto sub_score = [&](const typename Tile::Sub& k) {
    f32x4_t acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const u32x4_t bk = Tile::operand(k, kb);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt] = mfma_bf16_16x16x32(qa[mt][kb], bk, acc[mt]);
    }
    // Every product this lane holds belongs to its key c, whose fp8 scale s is one number, and
    // relu(s x) = s relu(x) for s >= 0: the scale multiplies the lane's sum once. A sub-tile
    // with a negative scale (the cache writer never makes one) takes the product per element.
    float p = 0.f;
    if (!FP8 || __ballot(k.sc < 0.f) == 0) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) p = fmaf(wv[mt][r], relu_f32(acc[mt][r]), p);
      if constexpr (FP8) p *= k.sc;
    } else {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) p = fmaf(wv[mt][r], relu_f32(acc[mt][r] * k.sc), p);
    }
    return p;
  };
  // the tile's four sub-tile shares -> candidate s0 + lane (reduce-scatter over the 4 lane
  // groups: group g keeps the full sum of sub-tile g), stored with its histogram count
  auto finish_tile = [&](const float* part, int s0) {
    const float total = reduce_scatter_rows4(part[0], part[1], part[2], part[3]);
    const int s = s0 + lane;
    if (s < n) {
      a.logits[(int64_t)t * a.ld_logits + s] = total;
      if constexpr (HIST) atomicAdd(&s_hist[float_key(total) >> (32 - kHistBits)], 1u);
    }
  };
  // Steady state (a next tile exists): the next tile's slots from the entries read one tile
  // ago, the entries of the tile after it (positions past the row read its last entry, so the
  // read needs no branch), then each sub-tile computed and refilled with the next tile's.
  // WHOLE: the next tile's entry comes from a register (the wave read the entries of 64 steps
  // at once), so no table read waits between key loads.
  int step = 0;
  while (tile + stride < ntiles) {
    int64_t sl[4];
    if constexpr (WHOLE) {
      ++step;
      if ((step & 63) == 0) ent = entries(b, step, n);   // the next 64 steps' entries (uniform)
      whole_slots(tile + stride, __builtin_amdgcn_readlane(ent, step & 63), sl);
    } else {
      Tile::finish(a, ad, sl);
      Tile::table(a, b, (tile + 2 * stride) << 6, n, c, ad);
    }
    __builtin_amdgcn_sched_barrier(0);   // the table reads stay ahead of the key loads
    float part[4];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      part[st] = sub_score(ring[st]);
      Tile::load(a, sl[st], g, ring[st]);
    }
    finish_tile(part, tile << 6);
    tile += stride;
  }
  if (tile < ntiles) {                   // the wave's last tile
    float part[4];
#pragma unroll
    for (int st = 0; st < 4; ++st) part[st] = sub_score(ring[st]);
    finish_tile(part, tile << 6);
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
  // tiles inside one page: one table entry per tile, read 64 steps at a time
  const bool whole = a.pg.bt ? a.pg.page % 64 == 0 : true;
  if (whole) launch_kernel(k_index_scores<DI, MT, FP8, HIST, true>, dim3(gx, T), dim3(kScoreThreads), st, a);
  else launch_kernel(k_index_scores<DI, MT, FP8, HIST, false>, dim3(gx, T), dim3(kScoreThreads), st, a);
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
