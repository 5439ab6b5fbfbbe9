// Sparse absorbed-MLA attention over gathered latent rows, gfx950 MFMA.
//
// For query row t and head h, over the listed cache rows c_i (entries -1 contribute nothing):
//   out[t,h] = sum_i softmax_i(softmax_scale * q[t,h] . c_i) * c_i[0:512],  lse = ln sum_i e^(.)
// Rows are 512 latent + 64 RoPE bf16 (tokenspeed PR 664 "gfx950 Gluon bf16 MLA decode and
// prefill kernels"), or fp8 rows of aiter PR 4382 "Paged Sparse Attention Gluon Kernel"
// (uniform pool: fp8 * fp32 scale per 64 columns, the bytes OCP or fnuz e4m3 (section "fp8
// flavors"; fnuz has no native conversion and is decoded by bit placement); fp8_ds_mla: 448 NoPE fp8 * 2^(e-127) per 64
// columns + 64 RoPE bf16, page-planar 584 bytes/token). -1 entries contribute nothing
// (radixark/miles PR 3608, "What", padding): they are dropped when a pass of the list is
// resolved to cache slots, so their rows are never read and they cost no blocks.
// A second list (extra) into a second cache shares the softmax (PR 4382, two-loop layout).
//
// Workgroup = HT x WD waves sharing each gathered 32-row block: a wave owns 16 heads (one of
// HT head tiles) and 512 / WD value columns (decode runs one head tile with WD = 4, so four
// waves issue the gather and the PV product and the score product is split over the waves).
// 64 heads (HT = 4, WD = 2: 8 waves) take 32x32x16 MFMAs for the value product instead: wave w
// owns 128 value columns (quarter w >> 1) of the 32 heads of half w & 1, and a 16-row x 16-head
// tile of the score product over the whole contraction, whose softmax it runs and whose packed
// weights it publishes; every wave of the head half then reads them as its P^T operand. About
// 240 registers per wave, so two waves share each SIMD. Each wave issues its share of the next
// block's row loads at its own point of the score product, so that the eight shares reach the
// CU's memory path one after another.
// Blocks stream through a ring of NBUF buffers in LDS: while a block is computed, the next
// NBUF - 1 blocks' rows are in flight (direct global->LDS loads; bf16 rows land in place, fp8
// rows land as raw bytes; fp8_ds_mla rows under one 16-head tile are converted straight into
// the MFMA operands, other fp8 rows are dequantised to one bf16 block just before use). Each
// wave waits only for its own loads of the block it needs (vmcnt = the loads of the later
// blocks), so the barriers never drain the ring. Every launch plan takes NBUF = 2 (deeper
// rings measured slower: they cost the second resident workgroup). Each wave computes
//   S^T[32 rows x 16 heads] = K Q^T   (A = rows from LDS, B = q held in registers),
// an online softmax in base 2, and
//   O^T[512 x 16 heads] += V^T P^T   (A = V^T read from LDS and transposed 8x8 in registers,
//                                      B = P^T straight from S^T's accumulator layout).
// With the 16x16x32 layout, S^T's accumulator rows (4 per lane group, two 16-row tiles) are
// exactly the k-slots of P^T as a B operand, so P never crosses lanes.
// The softmax runs in base 2 with a lazily rescaled running max. Splits (decode): each
// workgroup covers rows_per_split entries of the row's list and writes an un-normalised
// partial (o, m, l); k_mla_combine merges them (split-KV + LSE merge of PR 664).
// DeepSeek-V4 options (radixark/miles PR 3608, section "What", forward bullet: the lse the
// backward takes is in base 2 with the sink folded in): a per-head sink logit joins the
// softmax denominator only (it carries no value row), and the lse may be written in base 2.
#include "common.hpp"
#include "kernels.hpp"

namespace dsa {

constexpr int kNB = 32;     // rows per block
constexpr int kResolve = 1024;   // list entries resolved to slots per pass (multiple of kNB)
constexpr int kDV = 512;    // value width

// The reads of a block's rows: the score product's, 16 rows at one 16-byte column per 16
// lanes; the value product's, 64 bytes of each of 8 consecutive rows (transposing, 64-head
// path) or 256 bytes of rows 4 apart (16-head path). At this stride with row_swz (see there)
// none of them has a bank conflict. (Padding by 8 elements cost 4 conflict cycles per score
// read, by 16 none there but 2 per transposing read.)
template <int FMT, int DQK>
struct RowGeom {
  static constexpr int kElems = DQK + 32;                      // padded bf16 row in LDS
  static_assert((kElems * 2) % 128 == 64, "row stride");
  // 16-byte work units per row and what one unit produces
  static constexpr int kUnits = FMT == kFmtBf16 ? DQK / 8 : (kUniformFmt<FMT> ? DQK / 16 : 36);
};

// fp8 rows travel as raw bytes: data bytes per row (fp8_ds_mla: 448 fp8 + 64 bf16 RoPE; uniform
// pools: one byte per channel) and scale bytes per row (fp8_ds_mla: 7 UE8M0 + 1 pad; uniform:
// one fp32 per 64 channels)
template <int FMT, int DQK>
struct RawGeom {
  static constexpr int kData = FMT == kFmtDsMla ? 576 : DQK;
  static constexpr int kScale = FMT == kFmtDsMla ? 8 : (DQK / 64) * 4;
};

// One 16-byte unit of an fp8 row and its scale, on the way to bf16.
struct RawUnit {
  u32x4_t v;
  float sc;
};

// Byte offsets of a cache row, resolved once per row: the data (and for fp8 the scales).
struct RowOff {
  int64_t data;
  int64_t scale;
};

template <int FMT, int DQK>
__device__ __forceinline__ RowOff row_offsets(const KvDev& kv, int64_t slot) {
  RowOff o;
  if constexpr (FMT == kFmtBf16) {
    o.data = slot * DQK * 2;
    o.scale = 0;
  } else if constexpr (kUniformFmt<FMT>) {
    o.data = slot * DQK;
    o.scale = slot * (DQK / 64) * 4;
  } else {  // fp8_ds_mla: page-planar layout
    const int P = kv.pg.page;
    int64_t page, pos;
    if (kv.pg.page_shift >= 0) { page = slot >> kv.pg.page_shift; pos = slot & (P - 1); }
    else { page = slot / P; pos = slot - page * P; }
    const int64_t pbase = page * (int64_t)P * 584;
    o.data = pbase + pos * 576;
    o.scale = pbase + (int64_t)P * 576 + pos * 8;
  }
  return o;
}

// unit u of a row into its LDS row lrow, whose chunks are swizzled by sw (row_swz of the row)
template <int FMT, int DQK>
__device__ __forceinline__ void store_unit(const RawUnit& r, int u, uint16_t* lrow, int sw) {
  const bool rope = FMT == kFmtDsMla && u >= 28;
  if (rope) {   // RoPE columns of fp8_ds_mla rows are bf16 already
    *reinterpret_cast<u32x4_t*>(lrow + 8 * ((56 + u - 28) ^ sw)) = r.v;
    return;
  }
  if constexpr (FMT == kFmtDsMla) {   // UE8M0 scale, a power of two: one scaled conversion per pair
    u32x4_t lo, hi;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      lo[2 * k] = fp8x2_to_bf16x2_pow2<false>(r.v[k], r.sc);
      lo[2 * k + 1] = fp8x2_to_bf16x2_pow2<true>(r.v[k], r.sc);
      hi[2 * k] = fp8x2_to_bf16x2_pow2<false>(r.v[2 + k], r.sc);
      hi[2 * k + 1] = fp8x2_to_bf16x2_pow2<true>(r.v[2 + k], r.sc);
    }
    *reinterpret_cast<u32x4_t*>(lrow + 8 * ((2 * u) ^ sw)) = lo;
    *reinterpret_cast<u32x4_t*>(lrow + 8 * ((2 * u) ^ sw) + 8) = hi;
    return;
  }
  float f[16];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if constexpr (FMT == kFmtFnuz) fnuz4_to_f32(r.v[k], f + 4 * k);
    else fp8x4_to_f32(r.v[k], f + 4 * k);
  }
  u32x4_t lo, hi;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (kUniformFmt<FMT>) {     // arbitrary fp32 scale: round to bf16
      lo[i] = pack_bf16_rne(f[2 * i] * r.sc, f[2 * i + 1] * r.sc);
      hi[i] = pack_bf16_rne(f[8 + 2 * i] * r.sc, f[8 + 2 * i + 1] * r.sc);
    } else {                              // power-of-two scale: exact in bf16
      lo[i] = pack_bf16_exact(f[2 * i] * r.sc, f[2 * i + 1] * r.sc);
      hi[i] = pack_bf16_exact(f[8 + 2 * i] * r.sc, f[8 + 2 * i + 1] * r.sc);
    }
  }
  *reinterpret_cast<u32x4_t*>(lrow + 8 * ((2 * u) ^ sw)) = lo;
  *reinterpret_cast<u32x4_t*>(lrow + 8 * ((2 * u) ^ sw) + 8) = hi;
}

// Final normalisation of one (row, head) from its base-2 running max m and sum l (l = 0: no
// listed row), with the optional sink logit (natural-log units) in the denominator:
// returns the factor for the accumulated output, and the lse in the requested base.
struct Finish {
  float inv;
  float lse;
};
__device__ __forceinline__ Finish finish_softmax(float m, float l, float sink, bool lse_log2) {
  Finish f;
  float lse2;
  if (sink > -INFINITY) {
    const float s2 = sink * kLog2e;
    const float mm = fmaxf(m, s2);
    const float wl = l > 0.f ? exp2f(m - mm) : 0.f;   // weight of the listed rows' terms
    const float z = l * wl + exp2f(s2 - mm);
    f.inv = wl / z;
    lse2 = mm + log2f(z);
  } else {
    f.inv = l > 0.f ? 1.f / l : 0.f;
    lse2 = l > 0.f ? m + log2f(l) : -INFINITY;
  }
  f.lse = lse_log2 ? lse2 : lse2 * kLn2;
  return f;
}

// One direct global->LDS load (16 bytes per lane; lane l lands at lds_addr + 16 l) that the
// compiler does not see as one. Issued through the builtin, every later transposing LDS read
// waits for all such loads in flight (the compiler cannot tell them apart from the rows it
// reads). Here the kernel's own waits (vmcnt on the loads of the block it reads, then a
// barrier) order them. The load has no register result; M0 carries the LDS address (one wait
// state after it is written).
__device__ __forceinline__ void lds_dma16(const uint8_t* gptr, uint32_t lds_addr) {
  // (the address is the same in every lane; said so, or the compiler may hold it in a VGPR)
  const uint32_t lds_s = __builtin_amdgcn_readfirstlane(lds_addr);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(gptr), "s"(lds_s) : "m0");
}

template <int FMT, int DQK, int HT, int WD, bool SPLIT, int NBUF>
__global__ __launch_bounds__(64 * HT * WD, (HT == 1 || (HT == 4 && WD == 2)) ? 2 : 1) void k_sparse_mla(MlaArgs a) {
  static_assert(NBUF >= 2 && NBUF <= 4, "ring depth");
  constexpr int NW = HT * WD;                 // waves: HT head tiles x WD value-column slices
  constexpr int NT = 64 * NW;
  constexpr int GD = 4 / WD;                  // 128-column groups of the value a wave owns
  constexpr int KS = DQK / 32;
  constexpr int RE = RowGeom<FMT, DQK>::kElems;
  constexpr int UN = RowGeom<FMT, DQK>::kUnits;
  // bf16 rows: NBUF gathered blocks in LDS. fp8 rows: one bf16 block, plus NBUF raw blocks
  // (bytes as stored, data then scales) that the direct loads fill ahead of use
  constexpr bool kRaw = FMT != kFmtBf16;
  // fp8_ds_mla with one head tile and four waves: no bf16 block; the score and value products
  // convert their operands straight from the raw bytes (the scaled conversion is exact for
  // the power-of-two scales), which saves the LDS-to-LDS pass and its barrier
  constexpr bool kDirect = FMT == kFmtDsMla && HT == 1 && WD == 4;
  constexpr int BB = kNB * RE * 2;                            // bytes of one bf16 block
  constexpr int RDB = RawGeom<FMT, DQK>::kData;
  constexpr int RSB = RawGeom<FMT, DQK>::kScale;
  constexpr int RAWB = kNB * (RDB + RSB);                     // bytes of one raw block
  constexpr int RAW0 = kDirect ? 0 : BB;                      // offset of the raw ring
  constexpr int LDSB = kDirect ? NBUF * RAWB : (kRaw ? BB + NBUF * RAWB : NBUF * BB);
  static_assert(RDB % 16 == 0 && RSB % 4 == 0 && (kNB * RDB) % 1024 == 0, "raw staging");
  __shared__ __align__(16) uint8_t s_lds[LDSB];
  uint16_t (*const s_rows)[kNB][RE] = reinterpret_cast<uint16_t (*)[kNB][RE]>(s_lds);
  // list entries of the current pass resolved to cache slots: slot | list << 30, -1 = padding
  __shared__ __align__(16) int32_t s_slot[kResolve];

  const int t = blockIdx.z;
  const int hg = blockIdx.y;
  const int split = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int ht = wave % HT;                   // head tile of this wave
  const int gd0 = (wave / HT) * GD;           // first 128-column group of this wave
  const int g = lane >> 4;
  const int c = lane & 15;
  const int b = min(max(a.row_req ? a.row_req[t] : t, 0), a.n_req - 1);
  const int head0 = (hg * HT + ht) * 16;
  // The kernel-argument arrays are never indexed with a per-lane value (that becomes a
  // vector load from kernarg memory plus a full vmcnt wait, serialising the gathers).
  const KvDev kv0 = a.kv[0], kv1 = a.kv[1];
  const int32_t* const idx0 = a.idx[0];
  const int32_t* const idx1 = a.idx[1];
  const int64_t ld0 = a.ld_idx[0], ld1 = a.ld_idx[1];
  const int n0 = a.n_idx[0];
  const int ntot = n0 + a.n_idx[1];
  const int u_begin = split * a.rows_per_split;
  const int u_end = min(ntot, u_begin + a.rows_per_split);
  static_assert(kResolve % NT == 0 && kResolve % kNB == 0, "resolve pass");
  int pass_n = 0;   // listed rows of the current pass (slot table rows at or past it are padding)
  constexpr int RPT = kResolve / NT;
  __shared__ uint32_t s_cnt[RPT * NW];   // listed rows per (entry group, wave) of a pass

  // Entries [p0, p1) of the split (at most kResolve) to slots, all at once: every index read
  // of the thread, then every table read, then the slots (two round trips per pass instead
  // of two per block). Padding entries (-1) are dropped from passes longer than two blocks:
  // the listed rows are packed to the front of the slot table in list order (a ballot per
  // wave and entry group, their counts through LDS), so that blocks hold listed rows only and
  // a list padded with -1 costs no blocks for its padding. Returns the number of table rows
  // to process; the table reads -1 past them (and at padding entries of a short pass).
  auto resolve_pass = [&](int p0, int p1) -> int {
    int e[RPT];
    bool li[RPT];
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
      const int uu = min(p0 + (int)threadIdx.x + k * NT, p1 - 1);
      li[k] = uu >= n0;
      const int32_t* ip = li[k] ? idx1 + (int64_t)t * ld1 + (uu - n0) : idx0 + (int64_t)t * ld0 + uu;
      e[k] = *ip;
    }
    SlotRead sr[RPT];
#pragma unroll
    for (int k = 0; k < RPT; ++k) sr[k] = slot_read(pick_paging(li[k], kv1.pg, kv0.pg), b, max(e[k], 0));
    int32_t sv[RPT];
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
      const int j = threadIdx.x + k * NT;
      const int64_t slot = slot_done(pick_paging(li[k], kv1.pg, kv0.pg), sr[k]);
      sv[k] = j < p1 - p0 && e[k] >= 0 ? (int32_t)slot | ((int32_t)li[k] << 30) : -1;
    }
    // a pass of at most two blocks (a decode split) keeps its entries in place: packing could
    // save at most one block, less than the barrier and the LDS round trip it costs
    if (p1 - p0 <= 2 * kNB) {
#pragma unroll
      for (int k = 0; k < RPT; ++k) s_slot[threadIdx.x + k * NT] = sv[k];
      return p1 - p0;
    }
    uint64_t vm[RPT];
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
      vm[k] = __ballot(sv[k] >= 0);
      if (lane == 0) s_cnt[k * NW + wave] = (uint32_t)__popcll(vm[k]);
    }
    __syncthreads();
    uint32_t total = 0, before[RPT];
#pragma unroll
    for (int k = 0; k < RPT; ++k) before[k] = 0;
#pragma unroll
    for (int q = 0; q < RPT * NW; ++q) {
      const uint32_t cq = s_cnt[q];
#pragma unroll
      for (int k = 0; k < RPT; ++k) before[k] += q < k * NW + wave ? cq : 0u;
      total += cq;
    }
    const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
      const int j = threadIdx.x + k * NT;
      if (sv[k] >= 0) s_slot[before[k] + (uint32_t)__popcll(vm[k] & below)] = sv[k];
      // rows past the listed ones read as padding, so a block's row validity is its slot's sign
      if (j >= (int)total) s_slot[j] = -1;
    }
    // the same in every lane: said so, so that the block loop's bounds and waits stay scalar
    return __builtin_amdgcn_readfirstlane((int)total);
  };
  // cache row of pass entry j (a padding entry reads row 0 of the main cache: finite data,
  // masked by the softmax)
  // (j stays below kResolve: the read is unconditional, so that a thread's reads go out together
  // instead of one branch and one wait each)
  auto slot_at = [&](int j) -> int32_t {
    const int32_t v = s_slot[j];
    return j < pass_n ? v : -1;
  };
  auto row_of = [&](int j, bool& x) -> RowOff {
    const int32_t v = slot_at(j);
    x = v >= 0 && (v >> 30);
    const int64_t slot = v >= 0 ? (v & 0x3fffffff) : 0;
    return x ? row_offsets<FMT, DQK>(kv1, slot) : row_offsets<FMT, DQK>(kv0, slot);
  };
  // Source addresses of each row of the blocks in the ring (row data; fp8 scales), one slot
  // per ring buffer: computed once per row (one lane per row) an iteration before the
  // block's loads go out, so that the loads themselves need one LDS read and an add.
  __shared__ const uint8_t* s_ra[NBUF][kRaw ? 2 : 1][kNB];
  auto row_addrs = [&](int rs, int jb, int r) {    // row r of the block at pass entry jb
    bool x;
    const RowOff off = row_of(jb + r, x);
    const uint8_t* base = x ? kv1.data : kv0.data;
    s_ra[rs][0][r] = base + off.data;
    if constexpr (kRaw)
      s_ra[rs][1][r] = (FMT == kFmtDsMla ? base : reinterpret_cast<const uint8_t*>(x ? kv1.scales : kv0.scales)) + off.scale;
  };
  // bf16 rows into LDS by direct global->LDS loads (asynchronous, completes at the next vmcnt
  // wait)
  auto gather = [&](int buf) {   // the block in ring slot buf (addresses in s_ra[buf])
    if constexpr (FMT == kFmtBf16) {
      // lane l of instruction ins fills 16-byte slot 64 * ins + l of the padded block: chunk
      // cc ^ row_swz(r) of row r; the pad slots of each row re-read the row's first 64 bytes
      constexpr int RW = RE / 8;
      constexpr int SLOTS = kNB * RW;
      constexpr int NINS = (SLOTS + 63) / 64;
      constexpr int GI = NW;                           // issuing waves: all
      const int gw = wave;
      constexpr int PER = (NINS + GI - 1) / GI;        // instructions of a wave (at most)
      constexpr int BAT = PER > 6 ? (PER + 1) / 2 : PER;   // addresses read per batch
      auto* lbase = reinterpret_cast<__attribute__((address_space(3))) uint8_t*>(
          reinterpret_cast<uintptr_t>(&s_rows[buf][0][0]) & 0xffffffffu);
      {
#pragma unroll
        for (int k0 = 0; k0 < PER; k0 += BAT) {
          // a batch's address reads first (one LDS round trip), then its loads
          const uint8_t* src[BAT];
#pragma unroll
          for (int k = 0; k < BAT; ++k) {
            const int j = min((gw + (k0 + k) * GI) * 64 + lane, SLOTS - 1);
            const int r = j / RW;
            int cc = j - r * RW;
            cc = cc >= DQK / 8 ? cc - DQK / 8 : cc ^ row_swz(r);
            src[k] = s_ra[buf][0][r] + 16 * cc;
          }
#pragma unroll
          for (int k = 0; k < BAT; ++k) {
            const int ins = gw + (k0 + k) * GI;
            if (k0 + k < PER && ins < NINS && ins * 64 + lane < SLOTS) {
              // the builtin takes a named local: given an array element (or an expression over
              // the template-shaped address array) the host compilation silently drops the kernel
              const uint8_t* sp = src[k];
              __builtin_amdgcn_global_load_lds(sp, lbase + ins * 1024, 16, 0, 0);
            }
          }
        }
      }
    }
  };

  // 64 heads, bf16 rows: every wave issues its share of a block's loads at its own point of
  // the score product (wave w after k-step 2 w + 1), so that the waves find the CU's memory path
  // free in turn instead of all queueing on it at once (a load that finds it busy holds its
  // wave at issue): instruction k of this wave's share (its source, then its issue). Issued
  // as lds_dma16, since the builtin's loads would have to land before the value product.
  constexpr bool kStagger = FMT == kFmtBf16 && HT == 4 && WD == 2;
  constexpr int kGRW = RE / 8;                            // 16-byte slots per padded row
  constexpr int kGSlots = kNB * kGRW;
  constexpr int kGIns = (kGSlots + 63) / 64;               // instructions per block
  constexpr int kGPer = (kGIns + NW - 1) / NW;             // of one wave (at most)
  auto gsrc = [&](int buf, int k) -> const uint8_t* {
    const int j = min((wave + k * NW) * 64 + lane, kGSlots - 1);
    const int r = j / kGRW;
    int cc = j - r * kGRW;
    cc = cc >= DQK / 8 ? cc - DQK / 8 : cc ^ row_swz(r);
    return s_ra[buf][0][r] + 16 * cc;
  };
  auto gissue = [&](int buf, int k, const uint8_t* sp) {
    const int ins = wave + k * NW;
    const uint32_t lds = (uint32_t)(reinterpret_cast<uintptr_t>(&s_rows[buf][0][0]) & 0xffffffffu) + ins * 1024;
    if (ins < kGIns && ins * 64 + lane < kGSlots) lds_dma16(sp, lds);
  };

  // fp8 rows: the block's raw bytes go into raw buffer `buf` by direct global->LDS loads
  // (asynchronous; instruction ins of the data fills bytes [1024 ins, +1024), lane l at +16 l,
  // i.e. 16-byte chunk q = 64 ins + l = row q / (RDB / 16), chunk q % (RDB / 16); the scales
  // follow as dwords), one block ahead of its use
  auto gather_raw = [&](int buf) {   // the block in ring slot buf (addresses in s_ra[buf])
    uint8_t* rb = s_lds + RAW0 + buf * RAWB;
    auto* lds_d = reinterpret_cast<__attribute__((address_space(3))) uint8_t*>(reinterpret_cast<uintptr_t>(rb) & 0xffffffffu);
    auto* lds_s = lds_d + kNB * RDB;
    constexpr int CPR = RDB / 16;                    // 16-byte chunks per row
    constexpr int NID = kNB * RDB / 1024;            // data instructions per block
#pragma unroll
    for (int k = 0; k < (NID + NW - 1) / NW; ++k) {
      const int ins = wave + k * NW;
      if (ins < NID) {
        const int q = ins * 64 + lane;
        const int r = q / CPR;
        const uint8_t* sp = s_ra[buf][0][r] + 16 * (q - r * CPR);
        __builtin_amdgcn_global_load_lds(sp, lds_d + ins * 1024, 16, 0, 0);
      }
    }
    constexpr int SPR = RSB / 4;                     // scale dwords per row
    constexpr int NIS = (kNB * SPR + 63) / 64;       // scale instructions per block
#pragma unroll
    for (int k = 0; k < (NIS + NW - 1) / NW; ++k) {
      const int ins = wave + k * NW;
      const int q = ins * 64 + lane;
      if (ins < NIS && q < kNB * SPR) {
        const int r = q / SPR;
        const uint8_t* sp = s_ra[buf][kRaw ? 1 : 0][r] + 4 * (q - r * SPR);
        __builtin_amdgcn_global_load_lds(sp, lds_s + ins * 256, 4, 0, 0);
      }
    }
  };
  // raw buffer `buf` -> the bf16 block (LDS to LDS); list padding becomes zero rows
  // (the LDS reads of a batch of units go out before its first conversion; batches of three
  // keep the kernel at two waves per SIMD)
  auto dequant = [&](int buf, int jb) {
    const uint8_t* rb = s_lds + RAW0 + buf * RAWB;
    constexpr int QN = (kNB * UN + NT - 1) / NT;     // units per thread
    constexpr int QB = 3;                            // units per batch
#pragma unroll
    for (int q0 = 0; q0 < QN; q0 += QB) {
      RawUnit ru[QB];
#pragma unroll
      for (int q = 0; q < QB; ++q) {
        const int uid = min((int)threadIdx.x + (q0 + q) * NT, kNB * UN - 1);
        const int r = uid / UN;
        const int u = uid - r * UN;
        const uint8_t* rd = rb + r * RDB;
        const uint8_t* rs = rb + kNB * RDB + r * RSB;
        if constexpr (FMT == kFmtDsMla) {
          ru[q].v = *reinterpret_cast<const u32x4_t*>(rd + (u < 28 ? 16 * u : 448 + 16 * (u - 28)));
          ru[q].sc = u < 28 ? ue8m0_scale(rs[u >> 2]) : 0.f;
        } else {
          ru[q].v = *reinterpret_cast<const u32x4_t*>(rd + 16 * u);
          ru[q].sc = *reinterpret_cast<const float*>(rs + (u / 4) * 4);
        }
      }
#pragma unroll
      for (int q = 0; q < QB; ++q) {
        const int uid = threadIdx.x + (q0 + q) * NT;
        if (q0 + q < QN && uid < kNB * UN) {
          const int r = uid / UN;
          const int u = uid - r * UN;
          if (slot_at(jb + r) < 0) {
            ru[q].v = u32x4_t{0u, 0u, 0u, 0u};
            ru[q].sc = 0.f;
          }
          store_unit<FMT, DQK>(ru[q], u, &s_rows[0][r][0], row_swz(r));
        }
      }
    }
  };

  // The query heads (once per workgroup) are requested first, then the first pass's list
  // entries and table reads, so both round trips overlap; q is staged through the row
  // buffers (not yet in use).
  constexpr int QBYTES = HT * 16 * DQK * 2;
  constexpr int QIT = (QBYTES + NT * 16 - 1) / (NT * 16);
  // staged one head per padded row (RE elements): the 16 heads of one B-operand read then sit
  // in distinct LDS banks
  static_assert(HT * 16 * RE * 2 <= LDSB, "q staging");
  u32x4_t qreg[QIT];
  {
    // heads past H (a head count that is not a whole number of tiles) read as zero rows: their
    // scores are 0 and nothing of them is ever written
    const int qbytes = min(QBYTES, (a.H - hg * HT * 16) * DQK * 2);
    const uint8_t* qsrc = reinterpret_cast<const uint8_t*>(a.q + (int64_t)t * a.ld_q + (int64_t)(hg * HT * 16) * DQK);
#pragma unroll
    for (int i = 0; i < QIT; ++i) {
      const int o = (threadIdx.x + i * NT) * 16;
      qreg[i] = o < qbytes ? *reinterpret_cast<const u32x4_t*>(qsrc + o) : u32x4_t{0u, 0u, 0u, 0u};
    }
  }
  const int first_n = u_end > u_begin ? resolve_pass(u_begin, min(u_end, u_begin + kResolve)) : 0;
  {
    uint8_t* qdst = reinterpret_cast<uint8_t*>(&s_rows[0][0][0]);
#pragma unroll
    for (int i = 0; i < QIT; ++i) {
      const int o = (threadIdx.x + i * NT) * 16;
      const int h = o / (DQK * 2);   // staged like the rows: chunks swizzled by the head's row
      if (o < QBYTES) *reinterpret_cast<u32x4_t*>(qdst + h * (RE * 2) + 16 * (((o % (DQK * 2)) / 16) ^ row_swz(h))) = qreg[i];
    }
  }
  __syncthreads();
  // One head tile and four waves (decode): the waves split the score product instead of each
  // computing all of it, two per 16-row half of the block, each over half of the head
  // dimension; the four 16 x 16 partials meet in LDS. Every wave then holds the whole S^T.
  constexpr bool kSplitK = HT == 1 && WD == 4 && KS % 2 == 0;
  constexpr int KQ = kSplitK ? KS / 2 : KS;          // k-steps of the score product per wave
  const int kq0 = kSplitK ? (wave & 1) * KQ : 0;     // this wave's first k-step
  __shared__ f32x4_t s_sp[kSplitK ? 4 : 1][64];      // the partials
  // 64 heads (see the top): wave w belongs to head half hh = w & 1 and takes value slice
  // vh = w >> 1 (VC columns) of the half's 32 heads on 32x32x16 MFMAs (lane l: head 32 hh + l32,
  // k-slots 8 hl .. 8 hl + 7). Its score tile is 16 rows x 16 heads over the whole
  // contraction on 16x16x32 MFMAs: rows 16 rx .. + 15 and heads 16 hx .. + 15 of the half
  // (rx = vh & 1, hx = vh >> 1), so scores never cross waves; only the weights do.
  constexpr bool kW32 = HT == 4 && WD == 2;
  constexpr int NVS = 2 * WD;                         // waves per head half
  constexpr int VC = kDV / NVS;                       // value columns per wave
  constexpr int CPL = VC / 32;                        // columns per lane and row (m-tiles)
  static_assert(!kW32 || (NVS == 4 && CPL == 4), "32-head split");
  const int hh = wave & 1, vh = wave >> 1;
  const int l32 = lane & 31, hl = lane >> 5;
  const int rx = vh & 1, hx = vh >> 1;
  auto wv = [&](int r, int h) { return hh + 2 * (r + 2 * h); };   // the half's wave of tile (r, h)
  constexpr int PTS = 32 + 8;                         // padded row count of a head's weights (80-byte
                                                      // rows: the 8-byte reads of 32 heads conflict-free)
  __shared__ __align__(8) uint16_t s_pt[kW32 ? 2 : 1][32][PTS];   // P^T per half: [head][row], bf16
  __shared__ float s_mx[kW32 ? NW : 1][16];           // each wave's block max per score head
  __shared__ float s_lw[kW32 ? NW : 1][16];           // each wave's weight sum per score head (end)
  __shared__ __align__(8) uint8_t s_grow8[8];         // each wave's grow flag, in one word
  u32x4_t qb[KQ];
  if constexpr (kW32) {
    const uint16_t* qp = &s_rows[0][0][0] + (32 * hh + 16 * hx + c) * RE + 8 * (g ^ row_swz(c));
#pragma unroll
    for (int kb = 0; kb < KQ; ++kb) qb[kb] = *reinterpret_cast<const u32x4_t*>(qp + 32 * kb);
  } else {
    const uint16_t* qp = &s_rows[0][0][0] + (ht * 16 + c) * RE + 8 * (g ^ row_swz(c));
#pragma unroll
    for (int kb = 0; kb < KQ; ++kb) qb[kb] = *reinterpret_cast<const u32x4_t*>(qp + 32 * (kq0 + kb));
  }
  float m_run = -INFINITY;   // running max (base-2 units) of this lane's head; rescaled lazily
  float l_run = 0.f;         // lane-partial sum of exp2(s - m_run)
  // 64 heads: m_run and l_run belong to the lane's score head (16 hx + c of the half); m_o is
  // the same running max for the lane's value head (l32), kept in step with it
  float m_o = -INFINITY;
  f32x4_t o[kW32 ? 1 : GD][8];
  f32x16_t o32[kW32 ? CPL : 1];
#pragma unroll
  for (int i = 0; i < (kW32 ? 1 : GD); ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[i][e] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int e = 0; e < (kW32 ? CPL : 1); ++e) o32[e] = f32x16_t{};

  __syncthreads();   // q is in registers before the first rows land in the buffers
  // loads this wave issues per block (instructions of a block are dealt round-robin to the
  // waves; every one of them has at least one active lane, so each counts once on vmcnt)
  constexpr int NID = kNB * RDB / 1024;                      // raw data instructions
  constexpr int NIS = (kNB * (RSB / 4) + 63) / 64;           // raw scale instructions
  constexpr int NINS = (kNB * (RE / 8) + 63) / 64;           // bf16 instructions
  constexpr int PB_MAX = kRaw ? (NID + NW - 1) / NW + (NIS + NW - 1) / NW : (NINS + NW - 1) / NW;
  static_assert((NBUF - 2) * PB_MAX < 64, "vmcnt range");
  const int w_u = __builtin_amdgcn_readfirstlane(wave);
  const int per_block = kRaw ? (NID - w_u + NW - 1) / NW + (NIS - w_u + NW - 1) / NW
                             : (NINS - w_u + NW - 1) / NW;
  for (int p0 = u_begin; p0 < u_end; p0 += kResolve) {
    const int p1 = min(u_end, p0 + kResolve);
    if (p0 != u_begin) {
      __syncthreads();                   // every wave is done with the previous pass's slots
      pass_n = resolve_pass(p0, p1);
      __syncthreads();
    } else {
      pass_n = first_n;
    }
    const int nb = (pass_n + kNB - 1) / kNB;   // blocks of listed rows
    // the addresses of the first NBUF blocks (one thread per row), then the first NBUF - 1
    // blocks' loads
    for (int t = threadIdx.x; t < NBUF * kNB && t < nb * kNB; t += NT) row_addrs(t / kNB, (t / kNB) * kNB, t % kNB);
    // staggered loads: nothing of the list reads is left in flight (their values are in use),
    // but the compiler cannot prove it across the block loop and would wait for them there
    // with small counts that also cover the row loads it does not see
    if constexpr (kStagger) wait_vmcnt<0>();
    lds_barrier();
#pragma unroll
    for (int k = 0; k < NBUF - 1; ++k) {
      if (k < nb) {
        if constexpr (kRaw) {
          gather_raw(k);
        } else if constexpr (kStagger) {   // (no builtin LDS loads anywhere in this layout)
#pragma unroll
          for (int j = 0; j < kGPer; ++j) gissue(k, j, gsrc(k, j));
        } else {
          gather(k);
        }
      }
    }
  for (int it = 0; it < nb; ++it) {
    const int cur = kRaw ? 0 : it % NBUF;
    const int jb = it * kNB;             // pass entry of this block's first row
    // this block's rows (raw bytes for fp8) are in: the later blocks' loads stay in flight
    const int later = min(NBUF - 2, nb - 1 - it);
    wait_vmcnt_dyn<0, (NBUF - 2) * PB_MAX>(later * per_block);
    lds_barrier();                       // ... for every wave; and the buffer refilled below is free
    if (!kStagger && it + NBUF - 1 < nb) {
      if constexpr (kRaw) gather_raw((it + NBUF - 1) % NBUF);
      else gather((it + NBUF - 1) % NBUF);
    }
    // the addresses of the block after it, into the slot this block's loads used (read by
    // the next iteration's loads, after its barrier)
    if (it + NBUF < nb && threadIdx.x < kNB) row_addrs(it % NBUF, jb + NBUF * kNB, threadIdx.x);
    if constexpr (kRaw && !kDirect) {
      dequant(it % NBUF, jb);
      lds_barrier();                     // bf16 rows complete; the loads just issued stay in flight
    }
    // raw rows of this block (direct conversion): row r's data at rdb + r * RDB (448 fp8 NoPE
    // bytes then 64 bf16 RoPE values), its UE8M0 scale bytes at rsb + r * RSB
    const uint8_t* const rdb = s_lds + RAW0 + (it % NBUF) * RAWB;
    const uint8_t* const rsb = rdb + kNB * RDB;
    // 8 consecutive columns c0.. of raw row r as 8 bf16 (NoPE: 8 fp8 bytes times their group's
    // scale; RoPE: read as stored)
    auto raw8 = [&](int r, int c0) -> u32x4_t {
      const uint8_t* rd = rdb + r * RDB;
      if (c0 < 448) {
        const u32x2_t w = *reinterpret_cast<const u32x2_t*>(rd + c0);
        const float sc = ue8m0_scale(rsb[r * RSB + (c0 >> 6)]);
        return u32x4_t{fp8x2_to_bf16x2_pow2<false>(w[0], sc), fp8x2_to_bf16x2_pow2<true>(w[0], sc),
                       fp8x2_to_bf16x2_pow2<false>(w[1], sc), fp8x2_to_bf16x2_pow2<true>(w[1], sc)};
      }
      return *reinterpret_cast<const u32x4_t*>(rd + 448 + 2 * (c0 - 448));
    };

    // the block's row validity for the softmax (rows 4g..4g+3 and 16+4g..16+4g+3 of this lane),
    // read before the score product so the reads overlap it
    const int jm = jb + 4 * g;
    const u32x4_t sl0 = *reinterpret_cast<const u32x4_t*>(&s_slot[jm]);
    const u32x4_t sl1 = *reinterpret_cast<const u32x4_t*>(&s_slot[jm + 16]);

    if constexpr (kW32) {
      // ---- S^T tile: rows 16 rx + (lane & 15) of the block against this wave's 16 heads,
      // the whole contraction (A = rows from LDS, B = q in registers)
      f32x4_t sacc = f32x4_t{0.f, 0.f, 0.f, 0.f};
      {
        // operands read four k-steps ahead of their MFMA, so that no MFMA waits out a whole
        // LDS round trip (left to itself the compiler keeps one buffer and waits every step)
        const uint16_t* rp = &s_rows[cur][16 * rx + c][8 * (g ^ row_swz(c))];
        constexpr int DEPTH = 4;
        u32x4_t av[DEPTH];
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) av[d] = *reinterpret_cast<const u32x4_t*>(rp + 32 * d);
        const bool gnext = kStagger && it + NBUF - 1 < nb;
        const int gbuf = (it + NBUF - 1) % NBUF;
        static_assert(!kStagger || 2 * (NW - 1) + 1 < KQ, "every wave's turn inside the product");
#pragma unroll
        for (int kb = 0; kb < KQ; ++kb) {
          sacc = mfma_bf16_16x16x32(av[kb % DEPTH], qb[kb], sacc);
          if (kb + DEPTH < KQ) av[kb % DEPTH] = *reinterpret_cast<const u32x4_t*>(rp + 32 * (kb + DEPTH));
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // the MFMA,
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // then the next read
          if constexpr (kStagger) {
            if (gnext && kb == 2 * w_u + 1) {   // this wave's turn: its share of the next block
              const uint8_t* gs[kGPer];
#pragma unroll
              for (int k = 0; k < kGPer; ++k) gs[k] = gsrc(gbuf, k);
#pragma unroll
              for (int k = 0; k < kGPer; ++k) gissue(gbuf, k, gs[k]);
            }
          }
        }
      }
      // accumulator i of lane l: row 16 rx + 4 g + i, head 16 hx + c of the half
      const u32x4_t slv = *reinterpret_cast<const u32x4_t*>(&s_slot[jb + 16 * rx + 4 * g]);
      float x[4];
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[i] = (int32_t)slv[i] >= 0 ? sacc[i] * a.scale_log2 : -INFINITY;
        mx = fmaxf(mx, x[i]);
      }
      mx = max_xor32(max_xor16(mx));               // over the tile's 16 rows, per head
      // Weights against the running max, published as P^T (bf16) for the value product of
      // every wave of the half. They stand unless some wave's rows raise a head's max by more
      // than 2^8; then every wave rescales (its value heads and its score heads alike) and
      // publishes again.
      float p[4];
      auto weights = [&]() {
        const float m_use = m_run == -INFINITY ? 0.f : m_run;   // no valid row yet: x = -inf
#pragma unroll
        for (int i = 0; i < 4; ++i) p[i] = exp2_hw(x[i] - m_use);
        *reinterpret_cast<u32x2_t*>(&s_pt[hh][16 * hx + c][16 * rx + 4 * g]) =
            u32x2_t{pack_bf16_rne(p[0], p[1]), pack_bf16_rne(p[2], p[3])};
      };
      weights();
      const bool grow = __any(mx > m_run + 8.f);
      if (lane == 0) s_grow8[wave] = grow ? 1 : 0;
      if (g == 0) s_mx[wave][c] = mx;
      lds_barrier();
      // every wave's flag in one read, issued with the first k-step's weights (read again
      // below only if a rescale republishes them)
      const uint64_t flags = *reinterpret_cast<const uint64_t*>(s_grow8);
      u32x2_t pa0 = *reinterpret_cast<const u32x2_t*>(&s_pt[hh][l32][4 * hl]);
      u32x2_t pc0 = *reinterpret_cast<const u32x2_t*>(&s_pt[hh][l32][8 + 4 * hl]);
      const bool any_grow = flags != 0;
      if (any_grow) {                              // the same branch in every wave
        // a head's block max: the two row tiles of its head quarter
        const float bs = fmaxf(s_mx[wv(0, hx)][c], s_mx[wv(1, hx)][c]);
        const float bo = fmaxf(s_mx[wv(0, l32 >> 4)][l32 & 15], s_mx[wv(1, l32 >> 4)][l32 & 15]);
        const float ms_new = fmaxf(m_run, bs);
        const float mo_new = fmaxf(m_o, bo);
        if (m_o != -INFINITY) {
          const float alpha_o = exp2_hw(m_o - mo_new);
#pragma unroll
          for (int e = 0; e < CPL; ++e) o32[e] *= alpha_o;
        }
        if (m_run != -INFINITY) l_run *= exp2_hw(m_run - ms_new);
        m_run = ms_new;
        m_o = mo_new;
        weights();
        lds_barrier();
        pa0 = *reinterpret_cast<const u32x2_t*>(&s_pt[hh][l32][4 * hl]);
        pc0 = *reinterpret_cast<const u32x2_t*>(&s_pt[hh][l32][8 + 4 * hl]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) l_run += p[i];   // this lane's rows of its score head
      // ---- O^T += V^T P^T over this wave's VC value columns, two k-steps of 16 rows. k-slot
      // 8 hl + j of k-step ks is row 16 ks + 4 hl + j (j < 4) or 16 ks + 8 + 4 hl + j - 4: two
      // 8-byte reads of the value head's row of P^T. m-tile e is columns VC vh + 32 e .. + 31,
      // and its V^T operand comes from two transposing LDS reads (ds_read_b64_tr_b16): in each
      // 16-lane group, lane 4 a + b receives element b of the 4-column pieces that lanes a,
      // a + 4, a + 8, a + 12 address, so lane 16 G + 4 j + a addresses row 16 ks + 4 (G / 2) + j
      // (+ 8 for k-slots 4..7) at column 16 (G % 2) + 4 a of the tile, and every lane ends with
      // its column (lane % 32) of its 8 rows.
      {
        const int tg = lane >> 4, tj = (lane >> 2) & 3, ta = lane & 3;
        const int tr_row = 4 * (tg >> 1) + tj;
        const int tr_col = VC * vh + 16 * (tg & 1) + 4 * ta;
        const int tr_hi = (tg & 1) ? -16 : 16;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const u32x2_t pa = ks == 0 ? pa0 : *reinterpret_cast<const u32x2_t*>(&s_pt[hh][l32][16 + 4 * hl]);
          const u32x2_t pc = ks == 0 ? pc0 : *reinterpret_cast<const u32x2_t*>(&s_pt[hh][l32][24 + 4 * hl]);
          const u32x4_t pb = u32x4_t{pa[0], pa[1], pc[0], pc[1]};
#pragma unroll
          for (int e = 0; e < CPL; ++e) {
            // rows tr_row < 8 unswizzled, rows 8 + tr_row with chunk bit 1 flipped
            const uint16_t* rp = &s_rows[cur][16 * ks + tr_row][tr_col + 32 * e];
            const u32x2_t lo = ds_read_tr16(rp);
            const u32x2_t hi = ds_read_tr16(rp + 8 * RE + tr_hi);
            o32[e] = mfma_bf16_32x32x16(u32x4_t{lo[0], lo[1], hi[0], hi[1]}, pb, o32[e]);
          }
        }
      }
    } else {
    // ---- S^T = K Q^T
      f32x4_t s0 = f32x4_t{0.f, 0.f, 0.f, 0.f}, s1 = s0;
      if constexpr (kSplitK) {
        const uint16_t* rp = &s_rows[cur][16 * (wave >> 1) + c][8 * (g ^ row_swz(c)) + 32 * kq0];
        f32x4_t sp = s0;
  #pragma unroll
        for (int kb = 0; kb < KQ; ++kb) {
          if constexpr (kDirect)
            sp = mfma_bf16_16x16x32(raw8(16 * (wave >> 1) + c, 8 * g + 32 * (kq0 + kb)), qb[kb], sp);
          else
            sp = mfma_bf16_16x16x32(*reinterpret_cast<const u32x4_t*>(rp + 32 * kb), qb[kb], sp);
        }
        s_sp[wave][lane] = sp;
        lds_barrier();
        s0 = s_sp[0][lane] + s_sp[1][lane];
        s1 = s_sp[2][lane] + s_sp[3][lane];
      } else {
        const uint16_t* r0 = &s_rows[cur][c][8 * (g ^ row_swz(c))];
        const uint16_t* r1 = &s_rows[cur][16 + c][8 * (g ^ row_swz(c))];
  #pragma unroll
        for (int kb = 0; kb < KS; ++kb) {
          s0 = mfma_bf16_16x16x32(*reinterpret_cast<const u32x4_t*>(r0 + 32 * kb), qb[kb], s0);
          s1 = mfma_bf16_16x16x32(*reinterpret_cast<const u32x4_t*>(r1 + 32 * kb), qb[kb], s1);
        }
      }
      // ---- online softmax (base 2); the accumulators are rescaled only when some head's max
      // grows by more than 2^8, so exp2(s - m_run) stays <= 256
      float p[8];
      float mx = -INFINITY;
  #pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float x0 = (int32_t)sl0[r] >= 0 ? s0[r] * a.scale_log2 : -INFINITY;
        const float x1 = (int32_t)sl1[r] >= 0 ? s1[r] * a.scale_log2 : -INFINITY;
        p[r] = x0;
        p[4 + r] = x1;
        mx = fmaxf(mx, fmaxf(x0, x1));
      }
      mx = max_xor32(max_xor16(mx));
      if (__any(mx > m_run + 8.f)) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = m_run == -INFINITY ? 0.f : exp2_hw(m_run - m_new);
        if (m_run != -INFINITY || __any(l_run != 0.f)) {   // nothing to rescale before the first rows
          l_run *= alpha;
  #pragma unroll
          for (int i = 0; i < GD; ++i)
  #pragma unroll
            for (int e = 0; e < 8; ++e) o[i][e] *= alpha;
        }
        m_run = m_new;
      }
      const float m_use = m_run == -INFINITY ? 0.f : m_run;   // as in the 32-head path
  #pragma unroll
      for (int i = 0; i < 8; ++i) {
        p[i] = exp2_hw(p[i] - m_use);
        l_run += p[i];
      }
      u32x4_t pb;
      pb[0] = pack_bf16_rne(p[0], p[1]);
      pb[1] = pack_bf16_rne(p[2], p[3]);
      pb[2] = pack_bf16_rne(p[4], p[5]);
      pb[3] = pack_bf16_rne(p[6], p[7]);
      // ---- O^T += V^T P^T over this wave's value columns; V^T tiles come from 8 rows x 8
      // consecutive columns, transposed in registers
  #pragma unroll
      for (int i = 0; i < GD; ++i) {
        const int gd = gd0 + i;
        u32x4_t vr[8];
        if constexpr (kDirect) {
          // rows of list padding give zero values (their weights are zero, and their bytes, read
          // from slot 0, are not trusted to be finite)
  #pragma unroll
          for (int j = 0; j < 4; ++j) {
            const bool ok0 = jm + j < pass_n && (int32_t)sl0[j] >= 0;
            const bool ok1 = jm + 16 + j < pass_n && (int32_t)sl1[j] >= 0;
            const u32x4_t z = u32x4_t{0u, 0u, 0u, 0u};
            const u32x4_t v0 = raw8(4 * g + j, 128 * gd + 8 * c);
            const u32x4_t v1 = raw8(16 + 4 * g + j, 128 * gd + 8 * c);
            vr[j] = ok0 ? v0 : z;
            vr[4 + j] = ok1 ? v1 : z;
          }
        } else {
  #pragma unroll
          for (int j = 0; j < 4; ++j) {
            vr[j] = *reinterpret_cast<const u32x4_t*>(&s_rows[cur][4 * g + j][128 * gd + 8 * (c ^ row_swz(4 * g))]);
            vr[4 + j] = *reinterpret_cast<const u32x4_t*>(&s_rows[cur][16 + 4 * g + j][128 * gd + 8 * (c ^ row_swz(4 * g))]);
          }
        }
  #pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int w = e >> 1;
          const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
          u32x4_t av;
  #pragma unroll
          for (int pp = 0; pp < 4; ++pp) av[pp] = __builtin_amdgcn_perm(vr[2 * pp + 1][w], vr[2 * pp][w], sel);
          o[i][e] = mfma_bf16_16x16x32(av, pb, o[i][e]);
        }
      }
    }
  }
  }

  if constexpr (kW32) {
    // lane l holds head 32 hh + l32 (of the workgroup's 64), columns VC vh + 32 e + m for
    // m = 8 (r / 4) + 4 hl + r % 4 of accumulator r of m-tile e: four consecutive columns per
    // group of four accumulators. The weight sum of that head: each score lane's rows summed
    // over its tile's four row groups, then the head quarter's two row tiles
    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);
    if (g == 0) s_lw[wave][c] = l_run;
    __syncthreads();
    l_run = s_lw[wv(0, l32 >> 4)][l32 & 15] + s_lw[wv(1, l32 >> 4)][l32 & 15];
    m_run = m_o;
    const int headw = hg * 64 + 32 * hh + l32;
    const bool hv = headw < a.H;                        // not a padding head
    if constexpr (!SPLIT) {
      const Finish fin = finish_softmax(m_run, l_run, a.sink && hv ? a.sink[headw] : -INFINITY, a.lse_log2);
      uint16_t* op = a.out + (int64_t)t * a.ld_out + (int64_t)headw * kDV + VC * vh + 4 * hl;
#pragma unroll
      for (int e = 0; e < CPL; ++e)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const u32x2_t v = u32x2_t{pack_bf16_rne(o32[e][4 * q] * fin.inv, o32[e][4 * q + 1] * fin.inv),
                                    pack_bf16_rne(o32[e][4 * q + 2] * fin.inv, o32[e][4 * q + 3] * fin.inv)};
          if (hv) *reinterpret_cast<u32x2_t*>(op + 32 * e + 8 * q) = v;
        }
      if (a.lse && hv && hl == 0 && vh == 0) a.lse[(int64_t)t * a.H + headw] = fin.lse;
    } else {
      // The partial (o, m, l). A lane's pieces are 16 bytes scattered over 32 head rows, so
      // the block is staged in LDS (the ring is free: every wave is past the barrier above)
      // one head half at a time and written back one 2 KiB head row per 512 threads (whole
      // lines; as streaming stores they slowed the combine that reads them, 10.7 -> 12.6 us).
      constexpr int PS = kDV + 4;                       // padded fp32 row of one head in LDS
      static_assert(32 * PS * 4 <= LDSB, "partial staging");
      float* s_po = reinterpret_cast<float*>(s_lds);
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        if (half) __syncthreads();                      // the first half is written out
        if (hh == half) {
#pragma unroll
          for (int e = 0; e < CPL; ++e)
#pragma unroll
            for (int q = 0; q < 4; ++q)
              *reinterpret_cast<f32x4_t*>(s_po + l32 * PS + VC * vh + 32 * e + 8 * q + 4 * hl) =
                  f32x4_t{o32[e][4 * q], o32[e][4 * q + 1], o32[e][4 * q + 2], o32[e][4 * q + 3]};
        }
        __syncthreads();
        float* po = a.part_o + ((int64_t)t * a.Hp + hg * 64 + 32 * half) * a.n_split * kDV +
                    (int64_t)split * kDV;
        for (int q = threadIdx.x * 4; q < 32 * kDV; q += NT * 4) {
          const int hr = q / kDV;
          const int col = q - hr * kDV;
          *reinterpret_cast<f32x4_t*>(po + (int64_t)hr * a.n_split * kDV + col) =
              *reinterpret_cast<const f32x4_t*>(s_po + hr * PS + col);
        }
      }
      if (hl == 0 && vh == 0) {
        float* pml = a.part_ml + (((int64_t)t * a.Hp + headw) * a.n_split + split) * 2;
        pml[0] = m_run;
        pml[1] = l_run;
      }
    }
  } else {
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);

  const int head = head0 + c;
  const bool hv = head < a.H;                         // not a padding head
  if constexpr (!SPLIT) {
    const Finish fin = finish_softmax(m_run, l_run, a.sink && hv ? a.sink[head] : -INFINITY, a.lse_log2);
    const float inv = fin.inv;
    uint16_t* op = a.out + (int64_t)t * a.ld_out + (int64_t)head * kDV;
#pragma unroll
    for (int i = 0; i < GD; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        u32x4_t v;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2)
          v[e2] = pack_bf16_rne(o[i][2 * e2][r] * inv, o[i][2 * e2 + 1][r] * inv);
        if (hv) *reinterpret_cast<u32x4_t*>(op + 128 * (gd0 + i) + 32 * g + 8 * r) = v;
      }
    if (a.lse && hv && g == 0 && gd0 == 0) a.lse[(int64_t)t * a.H + head] = fin.lse;
  } else {
    // un-normalised partial (o, m, l) of this split; k_mla_combine merges them. A lane holds
    // 128 contiguous bytes of one head's row, so direct stores would spread every instruction
    // over 64 cache lines; the block is staged in LDS (free once every wave is past its last
    // block) and written back one head row at a time, 1 KiB per instruction, with streaming
    // (non-temporal) stores: whole lines that the next kernel reads (a streaming store of a
    // partial line, as the direct stores below would make, measured far slower).
    constexpr int PS = kDV + 4;                       // padded fp32 row of one head in LDS
    if constexpr (HT * 16 * PS * 4 <= LDSB) {
      float* s_po = reinterpret_cast<float*>(s_lds);
      lds_barrier();
#pragma unroll
      for (int i = 0; i < GD; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          f32x4_t v0, v1;
#pragma unroll
          for (int e = 0; e < 4; ++e) { v0[e] = o[i][e][r]; v1[e] = o[i][4 + e][r]; }
          float* d = s_po + (ht * 16 + c) * PS + 128 * (gd0 + i) + 32 * g + 8 * r;
          *reinterpret_cast<f32x4_t*>(d) = v0;
          *reinterpret_cast<f32x4_t*>(d + 4) = v1;
        }
      lds_barrier();
      float* po = a.part_o + ((int64_t)t * a.Hp + hg * HT * 16) * a.n_split * kDV + (int64_t)split * kDV;
      for (int q = threadIdx.x * 4; q < HT * 16 * kDV; q += NT * 4) {
        const int hl = q / kDV;
        const int col = q - hl * kDV;
        __builtin_nontemporal_store(*reinterpret_cast<const f32x4_t*>(s_po + hl * PS + col),
                                    reinterpret_cast<f32x4_t*>(po + (int64_t)hl * a.n_split * kDV + col));
      }
    } else {                                          // too many heads to stage: direct stores
      float* po = a.part_o + (((int64_t)t * a.Hp + head) * a.n_split + split) * kDV;
#pragma unroll
      for (int i = 0; i < GD; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          f32x4_t v0, v1;
#pragma unroll
          for (int e = 0; e < 4; ++e) { v0[e] = o[i][e][r]; v1[e] = o[i][4 + e][r]; }
          float* d = po + 128 * (gd0 + i) + 32 * g + 8 * r;
          *reinterpret_cast<f32x4_t*>(d) = v0;
          *reinterpret_cast<f32x4_t*>(d + 4) = v1;
        }
    }
    if (g == 0 && gd0 == 0) {
      float* pml = a.part_ml + (((int64_t)t * a.Hp + head) * a.n_split + split) * 2;
      pml[0] = m_run;
      pml[1] = l_run;
    }
  }
  }
}

// Merge the split partials of each (row, head): o = sum_s 2^(m_s - m) o_s / sum_s 2^(m_s - m) l_s
// (the LSE merge of PR 664). One 256-thread workgroup per (row, head, QW x 128 columns):
// groups of 32 QW threads (4 columns each) take every NG-th split, so each thread keeps
// several splits of loads in flight; the groups' sums meet in LDS. Many splits (a long row):
// QW = 1, eight groups, the work spread over many CUs. Few splits (many rows): QW = 4, a
// whole head per workgroup (a quarter-row workgroup would have one split per group).
template <int QW>
__global__ __launch_bounds__(256) void k_mla_combine(MlaArgs a) {
  constexpr int TPG = 32 * QW;                     // threads per split group
  constexpr int NG = 256 / TPG;                    // split groups
  __shared__ f32x4_t s_acc[NG][TPG];
  __shared__ float s_l[NG];
  __shared__ float s_m[NG];
  const int t = blockIdx.z;
  const int head = blockIdx.y;
  const int sg = threadIdx.x / TPG;
  const int ci = threadIdx.x % TPG;
  const int d0 = blockIdx.x * 128 * QW + ci * 4;
  const int S = a.n_split;
  const float* pml = a.part_ml + ((int64_t)t * a.Hp + head) * S * 2;
  const float* po = a.part_o + ((int64_t)t * a.Hp + head) * S * kDV + d0;
  // one pass: every partial (o, m, l) of this group's splits is requested at once and merged
  // online in registers (base-2 maxima); no separate pass for the global maximum
  float mg = -INFINITY, lg = 0.f;
  f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int sp0 = sg; sp0 < S; sp0 += NG * 8) {
    f32x4_t v[8];
    float m[8], l[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int sp = min(sp0 + u * NG, S - 1);
      v[u] = *reinterpret_cast<const f32x4_t*>(po + (int64_t)sp * kDV);
      m[u] = pml[2 * sp];
      l[u] = pml[2 * sp + 1];
    }
    float mx = mg;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (sp0 + u * NG >= S) m[u] = -INFINITY;
      mx = fmaxf(mx, m[u]);
    }
    if (mx != -INFINITY) {
      const float alpha = mg == -INFINITY ? 0.f : exp2f(mg - mx);
      acc *= alpha;
      lg *= alpha;
      mg = mx;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float wgt = m[u] == -INFINITY ? 0.f : exp2f(m[u] - mg);
        lg += wgt * l[u];
        acc += wgt * v[u];
      }
    }
  }
  s_acc[sg][ci] = acc;
  if (ci == 0) {
    s_l[sg] = lg;
    s_m[sg] = mg;
  }
  lds_barrier();
  if (sg != 0) return;
  float ms = -INFINITY;
#pragma unroll
  for (int q = 0; q < NG; ++q) ms = fmaxf(ms, s_m[q]);
  f32x4_t tot = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float lt = 0.f;
  if (ms != -INFINITY) {
#pragma unroll
    for (int q = 0; q < NG; ++q) {
      const float wgt = s_m[q] == -INFINITY ? 0.f : exp2f(s_m[q] - ms);
      tot += wgt * s_acc[q][ci];
      lt += wgt * s_l[q];
    }
  }
  const Finish fin = finish_softmax(ms, lt, a.sink ? a.sink[head] : -INFINITY, a.lse_log2);
  const float inv = fin.inv;
  uint16_t* op = a.out + (int64_t)t * a.ld_out + (int64_t)head * kDV + d0;
  u32x2_t vv;
  vv[0] = pack_bf16_rne(tot[0] * inv, tot[1] * inv);
  vv[1] = pack_bf16_rne(tot[2] * inv, tot[3] * inv);
  *reinterpret_cast<u32x2_t*>(op) = vv;
  if (a.lse && blockIdx.x == 0 && ci == 0) a.lse[(int64_t)t * a.H + head] = fin.lse;
}

template <int FMT, int DQK, int HT, int WD, int NBUF>
static hipError_t launch_h(const MlaArgs& a, int T, hipStream_t st) {
  dim3 grid(a.n_split, a.Hp / (16 * HT), T);
  if (a.n_split > 1)
    launch_kernel(k_sparse_mla<FMT, DQK, HT, WD, true, NBUF>, grid, dim3(64 * HT * WD), st, a);
  else
    launch_kernel(k_sparse_mla<FMT, DQK, HT, WD, false, NBUF>, grid, dim3(64 * HT * WD), st, a);
  return hipGetLastError();
}

// ht head tiles per workgroup (ht == 1 splits the value columns over 4 waves instead). Every
// plan takes a ring of two blocks (nbuf): deeper rings measured slower once a second
// workgroup per CU, or the 32-head layout, hides the gathers (the kernel keeps the parameter).
template <int FMT, int DQK>
static hipError_t launch_d(const MlaArgs& a, int ht, int nbuf, int T, hipStream_t st) {
  (void)nbuf;
  if (ht == 4) return launch_h<FMT, DQK, 4, 2, 2>(a, T, st);
  if (ht == 2) return launch_h<FMT, DQK, 2, 2, 2>(a, T, st);
  return launch_h<FMT, DQK, 1, 4, 2>(a, T, st);
}

hipError_t launch_sparse_mla(const MlaArgs& a, int fmt, int d_qk, int ht, int nbuf, int T, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  if (fmt == kFmtBf16) {
    if (d_qk == 576) return launch_d<kFmtBf16, 576>(a, ht, nbuf, T, st);
    return launch_d<kFmtBf16, 512>(a, ht, nbuf, T, st);
  }
  if (fmt == kFmtUniform) {
    if (d_qk == 576) return launch_d<kFmtUniform, 576>(a, ht, nbuf, T, st);
    return launch_d<kFmtUniform, 512>(a, ht, nbuf, T, st);
  }
  if (fmt == kFmtFnuz) {
    if (d_qk == 576) return launch_d<kFmtFnuz, 576>(a, ht, nbuf, T, st);
    return launch_d<kFmtFnuz, 512>(a, ht, nbuf, T, st);
  }
  return launch_d<kFmtDsMla, 512>(a, ht, nbuf, T, st);
}

hipError_t launch_mla_combine(const MlaArgs& a, int T, hipStream_t st) {
  if (T <= 0 || a.n_split <= 1) return hipSuccess;
  if (a.n_split <= 16)
    launch_kernel(k_mla_combine<4>, dim3(kDV / 512, a.H, T), dim3(256), st, a);
  else
    launch_kernel(k_mla_combine<1>, dim3(kDV / 128, a.H, T), dim3(256), st, a);
  return hipGetLastError();
}

}  // namespace dsa
