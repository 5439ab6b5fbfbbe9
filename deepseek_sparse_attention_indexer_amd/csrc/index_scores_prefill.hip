// Lightning-indexer scores for query rows that share their keys (causal or packed prefill,
// several query tokens per request), on gfx950 MFMA.
//
//   I(t, s) = index_scale * sum_j w[t, j] * max(0, q_idx[t, j, :] . k[slot(b, s), :])
//
// (the scoring stage of tokenspeed PR 627 "Add gluon kernel for DSA", prefill columns of its
// benchmark table, where scoring is the largest stage at long sequence lengths.)
//
// Per query row this is a [heads x di] x [di x keys] contraction followed by a ReLU-weighted
// head reduction. One query row per workgroup (the decode kernel) re-reads every key tile
// for every row, which makes a long causal prefill L2-bandwidth bound. Here a workgroup
// takes 4 consecutive rows (one per wave, all heads held in registers as MFMA A operands) and
// a chunk of up to 8192 key positions; each 64-key tile is read from memory once into a
// double-buffered LDS tile and used by all 4 rows. Two such workgroups share a CU (registers
// allow two waves per SIMD); their barriers are independent, so one workgroup's MFMAs run
// while the other waits on LDS or a barrier. The tile is stored XOR-swizzled (16-byte
// chunk p of key row r at p ^ (r mod chunks-per-row)) so that the 16 lanes that read one
// column of 16 key rows hit distinct banks. The epilogue is the decode kernel's: ReLU and the
// head weights in fp32 on the accumulators, a reduce-scatter by three lane swaps, one
// coalesced store of 64 scores per row and tile.
//
// Rows of a block that belong to different requests are processed one request after the
// other (each with its own keys); rows of the same request share the tiles. A row writes
// only its visible positions s < n_t.
#include "common.hpp"
#include "kernels.hpp"

namespace dsa {

constexpr int kPfRows = 4;                      // query rows per workgroup, one per wave
constexpr int kPfThreads = 64 * kPfRows;
constexpr int kPfTile = 64;                     // keys per LDS tile
constexpr int kPfChunkMax = 8192;               // key positions per workgroup (grid x), at most

template <int DI, int MT>
__global__ __launch_bounds__(kPfThreads, 2) void k_index_scores_prefill(ScoreArgs a, int T, int chunk) {
  constexpr int KB = DI / 32;                   // MFMA k-blocks of one key row
  constexpr int CPR = DI * 2 / 16;              // 16-byte chunks per key row
  constexpr int RB = DI * 2;                    // bytes per key row
  constexpr int TB = kPfTile * RB;              // bytes per tile
  constexpr int LPT = TB / (16 * kPfThreads);   // 16-byte loads per thread per tile
  static_assert(LPT >= 1 && TB % (16 * kPfThreads) == 0, "tile staging");
  __shared__ __align__(16) uint8_t s_k[2][TB];
  __shared__ int32_t s_slot[kPfChunkMax];
  __shared__ int32_t s_rowb[kPfRows];
  __shared__ int32_t s_rown[kPfRows];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4;
  const int c = lane & 15;
  // row blocks in reverse order: in a causal prefill the last rows see the most keys, and
  // starting the largest workgroups first keeps the end of the grid from waiting on them
  const int t = (gridDim.y - 1 - blockIdx.y) * kPfRows + wave;
  const bool row_ok = t < T;
  const int c0 = blockIdx.x * chunk;
  int my_n = 0;
  if (lane == 0) {
    int b = -1;
    if (row_ok) {
      b = min(max(a.row_req ? a.row_req[t] : t, 0), a.n_req - 1);
      my_n = min(max(a.row_len[t], 0), a.n_max);
    }
    s_rowb[wave] = b;
    s_rown[wave] = my_n;
  }
  lds_barrier();
  my_n = s_rown[wave];
  int blk_n = 0;
#pragma unroll
  for (int w = 0; w < kPfRows; ++w) blk_n = max(blk_n, s_rown[w]);
  if (blk_n <= c0) return;                      // no row of the block sees this chunk

  // this wave's query heads (A operands: qa[mt][kb] = q_idx[t, 16 mt + c, 32 kb + 8 g .. +7])
  // and the head weights of the accumulator rows it holds (head 16 mt + 4 g + r)
  u32x4_t qa[MT][KB];
  float wv[MT][4];
  {
    // unconditional loads from clamped addresses (a branch per load would put a wait after
    // each); out-of-range heads are zeroed afterwards
    const int tc = row_ok ? t : 0;
    const uint16_t* qrow = a.q_idx + (int64_t)tc * a.ld_q;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const int head = min(16 * mt + c, a.Hi - 1);
        qa[mt][kb] = *reinterpret_cast<const u32x4_t*>(qrow + head * DI + 32 * kb + 8 * g);
      }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) wv[mt][r] = a.w[(int64_t)tc * a.ld_w + min(16 * mt + 4 * g + r, a.Hi - 1)];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const bool qok = row_ok && 16 * mt + c < a.Hi;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        if (!qok) qa[mt][kb] = u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
      for (int r = 0; r < 4; ++r)
        wv[mt][r] = row_ok && 16 * mt + 4 * g + r < a.Hi ? wv[mt][r] * a.index_scale : 0.0f;
    }
  }

  uint32_t done = 0;                            // rows already processed (uniform)
  for (;;) {
    int w0 = -1;
#pragma unroll
    for (int w = kPfRows - 1; w >= 0; --w)
      if (!(done >> w & 1u) && s_rowb[w] >= 0) w0 = w;
    if (w0 < 0) break;
    const int b = s_rowb[w0];
    uint32_t grp = 0;
    int nmax = 0;
#pragma unroll
    for (int w = 0; w < kPfRows; ++w)
      if (s_rowb[w] == b) {
        grp |= 1u << w;
        nmax = max(nmax, s_rown[w]);
      }
    done |= grp;
    const int kend = min(c0 + chunk, nmax);
    if (kend <= c0) continue;
    const bool mine = grp >> wave & 1u;
    const int ntile = (kend - c0 + kPfTile - 1) / kPfTile;

    // slots of this request's keys in the chunk: every table read of the thread goes out at
    // once (a paged cache reads its block table, a packed one req_base[b]); positions past
    // kend are clamped and not stored
    for (int u0 = 0; u0 < kend - c0; u0 += 8 * kPfThreads) {
      const Paging& pg = a.pg;
      const bool paged = pg.bt != nullptr;
      const int32_t* tb = paged ? pg.bt : pg.req_base;
      int ent[8], offs[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int pos = c0 + min(u0 + (int)threadIdx.x + u * kPfThreads, kend - c0 - 1);
        const int q = pg.page_shift >= 0 ? (pos >> pg.page_shift) : pos / pg.page;
        const int lp = min(max(q, 0), max((int)pg.bt_stride - 1, 0));
        offs[u] = paged ? pos - q * pg.page : pos;
        ent[u] = tb[paged ? (int64_t)b * pg.bt_stride + lp : (int64_t)b];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = u0 + threadIdx.x + u * kPfThreads;
        const int64_t in_page = (int64_t)min(max(ent[u], 0), pg.n_pages - 1) * pg.page + offs[u];
        const int64_t v = (int64_t)ent[u] + offs[u];
        const int64_t packed = v < 0 ? 0 : (v >= pg.n_slots ? pg.n_slots - 1 : v);
        if (i < kend - c0) s_slot[i] = (int32_t)(paged ? in_page : packed);
      }
    }
    lds_barrier();

    // Tile j goes into LDS by direct global->LDS loads: instruction ins of the tile (1 KiB)
    // fills LDS bytes [1024 ins, 1024 ins + 1024) of the buffer, lane l at +16 l, i.e. chunk
    // position q = 64 ins + l = (key row r = q / CPR, position p = q % CPR); the lane fetches
    // global chunk p ^ (r % CPR) of that row, which stores the tile swizzled. Rows past the
    // request's last key re-read its last key (masked at the store). The loads complete on the
    // vector-memory counter, so the waits for them are explicit. The cache slots a tile's
    // loads need are read from LDS one tile ahead, so a tile's loads issue without waiting.
    constexpr int NINS = TB / 1024;
    constexpr int NPW = NINS / kPfRows;         // load instructions per wave and tile
    static_assert(NINS % kPfRows == 0, "whole instructions per wave");
    int slot_nx[NPW];
    // per load instruction k of this wave: the tile row its lane fetches and the swizzled
    // byte offset inside that row (the same for every tile); the wave index taken as uniform
    // so that each load's LDS destination is scalar arithmetic
    const int w_u = __builtin_amdgcn_readfirstlane(wave);
    int lrow[NPW], lswz[NPW];
#pragma unroll
    for (int k = 0; k < NPW; ++k) {
      const int q = (w_u + k * kPfRows) * 64 + lane;
      lrow[k] = q / CPR;
      lswz[k] = ((q % CPR) ^ (lrow[k] % CPR)) * 16;
    }
    auto read_slots = [&](int j) {
#pragma unroll
      for (int k = 0; k < NPW; ++k) slot_nx[k] = s_slot[min(j * kPfTile + lrow[k], kend - 1 - c0)];
    };
    auto dma_tile = [&](int buf) {
      auto* lbase = reinterpret_cast<__attribute__((address_space(3))) uint8_t*>(
          reinterpret_cast<uintptr_t>(&s_k[buf][0]) & 0xffffffffu);
#pragma unroll
      for (int k = 0; k < NPW; ++k) {
        const uint8_t* src = reinterpret_cast<const uint8_t*>(a.keys) + (uint64_t)(uint32_t)slot_nx[k] * RB + lswz[k];
        __builtin_amdgcn_global_load_lds(src, lbase + (w_u + k * kPfRows) * 1024, 16, 0, 0);
      }
    };
    read_slots(0);
    dma_tile(0);
    if (ntile > 1) read_slots(1);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier();

    auto mma = [&](const u32x4_t (&bv)[4][KB], int st, f32x4_t* acc) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt] = mfma_bf16_16x16x32(qa[mt][kb], bv[st][kb], acc[mt]);
    };
    auto epi = [&](const f32x4_t* acc) {
      float pp = 0.f;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) pp = fmaf(wv[mt][rr], relu_f32(acc[mt][rr]), pp);
      return pp;
    };
    // A tile's last sub-tile (accumulators acc1) is finished during the next tile's first
    // MFMAs: its epilogue, the reduce-scatter over the lane groups (lane l ends with the score
    // of key s0 + l) and the store.
    f32x4_t acc0[MT], acc1[MT];
    float part[4];
    auto finish = [&](int s0) {
      part[3] = epi(acc1);
      const float total = reduce_scatter_rows4(part[0], part[1], part[2], part[3]);
      const int s = s0 + lane;
      if (s < my_n && s < kend) a.logits[(int64_t)t * a.ld_logits + s] = total;
    };
    auto advance = [&](int j) {                 // loads of tile j + 1, slots of tile j + 2
      if (j + 1 < ntile) {
        dma_tile((j & 1) ^ 1);                  // that buffer was last read a tile ago
        if (j + 2 < ntile) read_slots(j + 2);
      }
    };
    // the wave scores tiles [0, jh) (its row sees them), then only loads and waits with the
    // others; the next tile's loads are complete before each barrier, while a store issued
    // after them (vector memory operations complete in issue order) may still be in flight
    const int jh = mine ? min(ntile, max(0, (my_n - c0 + kPfTile - 1) / kPfTile)) : 0;
    for (int j = 0; j < jh; ++j) {
      advance(j);
      const int cur = j & 1;
      // every B operand of the tile is read from LDS up front, so the MFMAs run back to back
      u32x4_t bv[4][KB];
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const int r = 16 * st + c;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const int cc = 4 * kb + g;
          bv[st][kb] = *reinterpret_cast<const u32x4_t*>(&s_k[cur][r * RB + ((cc ^ (r % CPR)) * 16)]);
        }
      }
      // the MFMAs of sub-tile st + 1 are issued before the epilogue of sub-tile st, so the
      // matrix cores run while the vector ALU applies ReLU and the head weights
      mma(bv, 0, acc0);
      if (j > 0) finish(c0 + (j - 1) * kPfTile);
      mma(bv, 1, acc1);
      part[0] = epi(acc0);
      mma(bv, 2, acc0);
      part[1] = epi(acc1);
      mma(bv, 3, acc1);
      part[2] = epi(acc0);
      if (j > 0) asm volatile("s_waitcnt vmcnt(1)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      lds_barrier();
    }
    for (int j = jh; j < ntile; ++j) {
      advance(j);
      if (j == jh && jh > 0) {
        finish(c0 + (jh - 1) * kPfTile);
        asm volatile("s_waitcnt vmcnt(1)" ::: "memory");
      } else {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
      lds_barrier();
    }
    if (jh == ntile && jh > 0) finish(c0 + (jh - 1) * kPfTile);
  }
}

template <int DI>
static hipError_t launch_prefill_di(const ScoreArgs& a, int T, hipStream_t st) {
  // the largest chunk that still gives about two workgroups per CU (few row blocks, e.g. an
  // extend chunk, need short chunks to fill the chip; a long prefill has rows enough)
  const int nrb = (T + kPfRows - 1) / kPfRows;
  int chunk = kPfChunkMax;
  while (chunk > 1024 && (int64_t)nrb * ((a.n_max + chunk - 1) / chunk) < 512) chunk >>= 1;
  const dim3 grid((a.n_max + chunk - 1) / chunk, nrb);
  if (a.Hi <= 16) launch_kernel(k_index_scores_prefill<DI, 1>, grid, dim3(kPfThreads), st, a, T, chunk);
  else if (a.Hi <= 32) launch_kernel(k_index_scores_prefill<DI, 2>, grid, dim3(kPfThreads), st, a, T, chunk);
  else launch_kernel(k_index_scores_prefill<DI, 4>, grid, dim3(kPfThreads), st, a, T, chunk);
  return hipGetLastError();
}

hipError_t launch_index_scores_prefill(const ScoreArgs& a, int di, int T, hipStream_t st) {
  if (T <= 0 || a.n_max <= 0) return hipSuccess;
  if (di == 64) return launch_prefill_di<64>(a, T, st);
  return launch_prefill_di<128>(a, T, st);
}

}  // namespace dsa
