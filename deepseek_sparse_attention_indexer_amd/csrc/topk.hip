// Per-row top-k of the indexer scores on gfx950.
//
// Output contract (decode top-k wrapper of tokenspeed PR 627 "Add gluon kernel for DSA",
// review: it returns (out, lens_out)): indices[t, 0:topk] hold the positions of the
// min(topk, n_t) largest scores in unspecified order, then -1; lens[t] = min(topk, n_t).
// Ties are broken toward the smaller position, so the selected SET is deterministic.
//
// Method: radix select on the order-preserving uint32 image of the fp32 scores, most
// significant digit first, counting with histograms (the threshold / greater / equal counting
// of the PR 627 selector). Digits are 12, 12 and 8 bits. When more candidates share the
// threshold key than slots remain, the ties are resolved by a second radix select on the
// complemented position. Output slots come from prefix sums of the selection counts, never
// from racing atomics, so the list's order is the same on every run.
//
//  * k_topk_lds: one 512-thread workgroup per row, the row's keys held in registers (<= 16K); the
//    list is in position order.
//  * long rows: the first-digit histogram is built per chunk (k_topk_hist, or fused into
//    the score kernel). k_topk_filter's workgroups (one per chunk) find the threshold bin and
//    write their chunk's threshold-bin candidates and counts. In k_topk_finalize one
//    workgroup per chunk writes the chunk's keys above the bin while one more workgroup per
//    row resolves the bin from its candidates (usually a few thousand, held in LDS). Kernel
//    boundaries replace device-scope fences and returning atomics, which cost microseconds
//    each on this part.
#include "common.hpp"
#include "kernels.hpp"
#include "select.hpp"

namespace dsa {

constexpr int kNT = 512;   // threads of the select workgroups

// ------------------------------------------------------------------ rows that fit in LDS
// CAP: key capacity (a multiple of the 512 threads). Key i of the row is held in register
// i / 512 of thread i % 512, so every pass over the keys (three radix digits, the ties, the
// compaction in position order) reads registers, and LDS holds only the 16 KiB histogram:
// up to four workgroups per CU. CAP = 8704 covers a causal prefill of 8K tokens plus a few.
template <int CAP>
__global__ __launch_bounds__(kNT) void k_topk_lds(TopkArgs a) {
  static_assert(CAP % kNT == 0, "whole registers");
  constexpr int PER = CAP / kNT;
  __shared__ uint32_t s_hist[kHistBins];
  __shared__ uint32_t s_w[kNT / 64];
  __shared__ uint32_t s_res[4];

  const int t = blockIdx.x;
  const int k = a.topk;
  int n = a.row_len[t];
  n = min(max(n, 0), a.n_max);
  int32_t* out = a.indices + (int64_t)t * a.ld_idx;
  if (n <= k) {
    for (int i = threadIdx.x; i < k; i += kNT) out[i] = i < n ? i : -1;
    if (threadIdx.x == 0) a.lens[t] = n;
    return;
  }
  const float* row = a.logits + (int64_t)t * a.ld_logits;
  // every load of the thread in flight at once, from clamped positions (a loop of load, wait,
  // store would pay one memory round trip per 512 keys); positions past n are never taken
  uint32_t key[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) key[j] = float_key(row[min((int)threadIdx.x + j * kNT, n - 1)]);
  auto valid = [&](int j) { return (int)threadIdx.x + j * kNT < n; };

  uint32_t need = (uint32_t)k, eq = 0;
  auto get_key = [&](int j, uint32_t& kk) { kk = key[j]; return valid(j); };
  const uint32_t thr = radix_select_regs<kNT, PER>(get_key, 0u, 0u, 32, need, &eq, s_hist, s_w, s_res);
  // ties at thr: keep the `need` smallest positions (largest complemented positions)
  uint32_t pos_thr = 0u;
  if (eq > need) {
    uint32_t need2 = need, eq2 = 0;
    auto get_tie = [&](int j, uint32_t& kk) {
      kk = ~(uint32_t)((int)threadIdx.x + j * kNT);
      return valid(j) && key[j] == thr;
    };
    pos_thr = radix_select_regs<kNT, PER>(get_tie, 0u, 0u, 32, need2, &eq2, s_hist, s_w, s_res);
  }
  const bool all_ties = eq <= need;
  // Compaction in position order, so the list (and everything computed from it in list order)
  // is the same on every run: the selected count of every (pass, wave) pair, one scan over
  // those counts (pass-major), then each lane writes at its pair's offset plus the selected
  // lanes below it. The histogram is free for the counts.
  constexpr int NW = kNT / 64;
  static_assert(PER * NW <= kNT && PER * NW <= kHistBins, "pair counts");
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  auto selected = [&](int j) {
    const uint32_t kk = key[j];
    const uint32_t i = (uint32_t)((int)threadIdx.x + j * kNT);
    return valid(j) && (kk > thr || (kk == thr && (all_ties || ~i >= pos_thr)));
  };
  bool sel[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    sel[j] = selected(j);
    const uint64_t m = __ballot(sel[j]);
    if (lane == 0) s_hist[j * NW + wv] = (uint32_t)__popcll(m);
  }
  lds_barrier();
  {
    const int j = threadIdx.x;
    const uint32_t c = j < PER * NW ? s_hist[j] : 0u;
    const uint32_t incl = block_incl_scan<kNT>(c, s_w, nullptr);
    lds_barrier();                             // every count read before the offsets replace them
    if (j < PER * NW) s_hist[j] = incl - c;
  }
  lds_barrier();
  const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const uint64_t m = __ballot(sel[j]);
    const uint32_t o = s_hist[j * NW + wv] + (uint32_t)__popcll(m & below);
    if (sel[j] && o < (uint32_t)k) out[o] = (int)threadIdx.x + j * kNT;
  }
  if (threadIdx.x == 0) a.lens[t] = k;
}

// ------------------------------------------------------------------ long rows
__global__ __launch_bounds__(kNT) void k_topk_hist(TopkArgs a) {
  __shared__ uint32_t s_hist[kHistBins];
  const int t = blockIdx.y;
  int n = a.row_len[t];
  n = min(max(n, 0), a.n_max);
  const int s0 = blockIdx.x * kTopkChunk;
  if (s0 >= n) return;
  // the chunk's scores requested before the histogram is cleared, all at once (clamped
  // positions; those past the row's end are not counted)
  const float* row = a.logits + (int64_t)t * a.ld_logits;
  const int s1 = min(n, s0 + kTopkChunk);
  constexpr int per = kTopkChunk / kNT;
  float v[per];
#pragma unroll
  for (int j = 0; j < per; ++j) v[j] = row[min(s0 + j * kNT + (int)threadIdx.x, s1 - 1)];
  for (int i = threadIdx.x; i < kHistBins; i += kNT) s_hist[i] = 0;
  lds_barrier();
#pragma unroll
  for (int j = 0; j < per; ++j)
    if (s0 + j * kNT + (int)threadIdx.x < s1) atomicAdd(&s_hist[float_key(v[j]) >> (32 - kHistBits)], 1u);
  lds_barrier();
  uint32_t* gh = a.hist + ((int64_t)t * kHistSlices + (blockIdx.x % kHistSlices)) * kHistBins;
  for (int i = threadIdx.x; i < kHistBins; i += kNT) {
    const uint32_t v = s_hist[i];
    if (v) atomicAdd(gh + i, v);
  }
}

// One workgroup per (row, chunk of kTopkChunk candidates). From the row's first-digit
// histogram it finds the threshold bin, then writes this chunk's threshold-bin candidates
// (key, position) into the chunk's own region and the chunk's counts (above the bin, in it).
// No returning atomics and no fences: the kernel boundary publishes everything.
__global__ __launch_bounds__(kNT) void k_topk_filter(TopkArgs a) {
  __shared__ uint32_t s_hist[kHistBins];
  __shared__ uint32_t s_w[kNT / 64];
  __shared__ uint32_t s_res[8];

  constexpr int D1 = 32 - kHistBits;          // shift of the first digit
  constexpr int per = kTopkChunk / kNT;
  const int t = blockIdx.y;
  const int k = a.topk;
  const int s0 = blockIdx.x * kTopkChunk;
  // this chunk's scores go out first, before the row length is known (positions below the
  // longest row stay inside the logits row); the histogram read overlaps them
  uint32_t keys[per];
  const float* row = a.logits + (int64_t)t * a.ld_logits;
  {
    // unconditional loads from clamped positions, all in flight together (a load under a
    // branch gets its wait inside the branch: one round trip per load)
    const int s1_max = min(a.n_max, s0 + kTopkChunk);
    float v[per];
#pragma unroll
    for (int j = 0; j < per; ++j) v[j] = row[min(s0 + j * kNT + (int)threadIdx.x, s1_max - 1)];
#pragma unroll
    for (int j = 0; j < per; ++j) {
      const int s = s0 + j * kNT + threadIdx.x;
      keys[j] = s < s1_max ? float_key(v[j]) : 0u;
    }
  }
  int n = a.row_len[t];
  n = min(max(n, 0), a.n_max);
  const int s1 = min(n, s0 + kTopkChunk);
  int32_t* out = a.indices + (int64_t)t * a.ld_idx;
  if (n <= k) {                                // every position is selected
    for (int s = s0 + threadIdx.x; s < s1; s += kNT) out[s] = s;
    return;
  }
  if (s0 >= n) return;
  const uint32_t* gh = a.hist + (int64_t)t * kHistSlices * kHistBins;
  {
    // every slice of every bin this thread sums is in flight at once (one round trip)
    constexpr int HB = kHistBins / kNT;
    uint32_t v[HB][kHistSlices];
#pragma unroll
    for (int h = 0; h < HB; ++h)
#pragma unroll
      for (int sl = 0; sl < kHistSlices; ++sl) v[h][sl] = gh[sl * kHistBins + h * kNT + threadIdx.x];
#pragma unroll
    for (int h = 0; h < HB; ++h) {
      uint32_t x = 0;
#pragma unroll
      for (int sl = 0; sl < kHistSlices; ++sl) x += v[h][sl];
      s_hist[h * kNT + threadIdx.x] = x;
    }
  }
  lds_barrier();
  find_digit_desc<kNT>(s_hist, kHistBins, (uint32_t)k, s_w, s_res);
  const uint32_t d1 = s_res[0];
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    a.thr1[2 * t] = d1;
    a.thr1[2 * t + 1] = s_res[1];
  }
  uint32_t n_gt = 0, n_eq = 0;
#pragma unroll
  for (int j = 0; j < per; ++j) {
    const int s = s0 + j * kNT + threadIdx.x;
    if (s < s1) {
      const uint32_t dg = keys[j] >> D1;
      n_gt += dg > d1;
      n_eq += dg == d1;
    }
  }
  // one scan for both counts: above the bin in the high 16 bits, in it in the low 16 (a chunk
  // holds kTopkChunk <= 65535 candidates, so the low half never carries into the high one)
  static_assert(kTopkChunk < 65536, "packed counts");
  uint32_t tot;
  const uint32_t inc = block_incl_scan<kNT>((n_gt << 16) | n_eq, s_w, &tot);
  const uint32_t tot_gt = tot >> 16, tot_eq = tot & 0xFFFFu;
  uint32_t o_eq = (inc & 0xFFFFu) - n_eq;
  const int64_t region = ((int64_t)t * a.n_chunks + blockIdx.x) * kTopkChunk;
  uint32_t* ck = a.cand_key + region;
  int32_t* cp = a.cand_pos + region;
#pragma unroll
  for (int j = 0; j < per; ++j) {
    const int s = s0 + j * kNT + threadIdx.x;
    if (s < s1 && (keys[j] >> D1) == d1) {
      ck[o_eq] = keys[j];
      cp[o_eq] = s;
      ++o_eq;
    }
  }
  if (threadIdx.x == 0) {
    uint32_t* cnt = a.counts + ((int64_t)t * a.n_chunks + blockIdx.x) * 2;
    cnt[0] = tot_gt;
    cnt[1] = tot_eq;
  }
}

// Per row: one workgroup per chunk writes the chunk's keys above the threshold bin, and one
// more workgroup (x == n_chunks) resolves the bin. Output layout: [keys above the bin, chunk
// by chunk] then [the bin's selected keys, in candidate order]; both orders are fixed, so the
// list is deterministic.
//  * chunk workgroups: offset = sum of the earlier chunks' counts above the bin, then a
//    thread-major scan of the chunk's own scores;
//  * the resolver: gathers the bin's candidates (up to 4096 held in registers, up to CAND
//    more in LDS, else re-read from the workspace), takes the second digit and the
//    threshold sub-bin's last 8 bits by histogram, breaks ties at the threshold key toward
//    the smaller position, then writes the selected candidates. It also returns the
//    first-digit histogram to zero, writes lens and pads short rows with -1.
// CAND: candidate capacity in LDS. The LDS of a kernel is reserved for every workgroup, so a
// large grid (many rows) takes CAND = 0: its chunk workgroups then fit four to a CU, and a
// row with more than 4096 candidates re-reads them from the workspace.
template <int CAND>
__global__ __launch_bounds__(kNT) void k_topk_finalize(TopkArgs a) {
  __shared__ uint32_t s_hist[kHistBins];
  __shared__ uint32_t s_w[kNT / 64];
  __shared__ uint32_t s_res[8];
  __shared__ uint32_t s_off[kMaxChunks + 1];   // the bin's candidates per chunk -> prefixes
  __shared__ uint32_t s_ck[CAND > 0 ? CAND : 1];   // candidate keys
  __shared__ int32_t s_cp[CAND > 0 ? CAND : 1];    // and positions

  constexpr int D1 = 32 - kHistBits;
  constexpr int D2 = D1 - kHistBits;
  constexpr int per = kTopkChunk / kNT;
  const int t = blockIdx.y;
  const int k = a.topk;
  int32_t* out = a.indices + (int64_t)t * a.ld_idx;
  const uint32_t* cnt = a.counts + (int64_t)t * a.n_chunks * 2;

  if ((int)blockIdx.x < a.n_chunks) {
    // ---- chunk workgroup: keys above the threshold bin. Its loads go out before the row
    // length is known (chunks past the row's end then simply return). Every chunk workgroup
    // first returns its share of the row's first-digit histogram to zero (all readers of it
    // ran in the previous kernel).
    const int c_me = blockIdx.x;
    const int s0 = c_me * kTopkChunk;
    {
      constexpr int HW = kHistSlices * kHistBins;
      const int share = (HW + a.n_chunks - 1) / a.n_chunks;
      uint32_t* gh = a.hist + (int64_t)t * HW;
      const int h1 = min(HW, (c_me + 1) * share);
      for (int i = c_me * share + threadIdx.x; i < h1; i += kNT) gh[i] = 0;
    }
    uint32_t before = 0;                       // counts of the earlier chunks
    for (int c = threadIdx.x; c < c_me; c += kNT) before += cnt[2 * c];
    uint32_t keys[per];
    const float* row = a.logits + (int64_t)t * a.ld_logits;
    {
      // (unconditional loads from clamped positions, all in flight together, as in the filter)
      const int s1_max = min(a.n_max, s0 + kTopkChunk);
      float v[per];
#pragma unroll
      for (int j = 0; j < per; ++j) v[j] = row[min(s0 + j * kNT + (int)threadIdx.x, s1_max - 1)];
#pragma unroll
      for (int j = 0; j < per; ++j) {
        const int s = s0 + j * kNT + threadIdx.x;
        keys[j] = s < s1_max ? float_key(v[j]) : 0u;
      }
    }
    const uint32_t d1 = a.thr1[2 * t];
    int n = a.row_len[t];
    n = min(max(n, 0), a.n_max);
    const int nch = (n + kTopkChunk - 1) / kTopkChunk;
    if (n <= k || c_me >= nch) return;
    const int s1 = min(n, s0 + kTopkChunk);
    uint32_t base;
    block_incl_scan<kNT>(before, s_w, &base);
    uint32_t sel = 0, m = 0;
#pragma unroll
    for (int j = 0; j < per; ++j) {
      const int s = s0 + j * kNT + threadIdx.x;
      const bool x = s < s1 && (keys[j] >> D1) > d1;
      sel |= (uint32_t)x << j;
      m += x;
    }
    uint32_t tot;
    uint32_t o = base + block_incl_scan<kNT>(m, s_w, &tot) - m;
#pragma unroll
    for (int j = 0; j < per; ++j)
      if (sel >> j & 1u) {
        if (o < (uint32_t)k) out[o] = s0 + j * kNT + threadIdx.x;
        ++o;
      }
    return;
  }

  // ---- the resolver: the per-chunk counts go out before the row length is known
  const int c0 = 2 * threadIdx.x;
  const uint32_t r0 = c0 < a.n_chunks ? cnt[2 * c0 + 1] : 0u;
  const uint32_t r1 = c0 + 1 < a.n_chunks ? cnt[2 * c0 + 3] : 0u;
  // Up to RU * kNT candidates stay in registers (kk, pp) for every later step. With at most
  // 64 chunks, the first SJ = 2^sj_log candidates of every chunk fill those slots exactly
  // (slot q = u * kNT + thread: chunk q >> sj_log, entry q & (SJ - 1)); they are requested
  // together with the counts, a round trip earlier than counts-then-candidates, and masked
  // once the counts are known. A chunk holding more than SJ (rare) takes the general path.
  constexpr int RU = 8;
  uint32_t kk[RU];
  int32_t pp[RU];
  const int sj_log = 31 - __clz((RU * kNT) / max(a.n_chunks, 1));   // uniform
  if (sj_log >= 6) {
#pragma unroll
    for (int u = 0; u < RU; ++u) {
      const int q = u * kNT + threadIdx.x;
      const int cc = min(q >> sj_log, a.n_chunks - 1);
      const int64_t at = ((int64_t)t * a.n_chunks + cc) * kTopkChunk + (q & ((1 << sj_log) - 1));
      kk[u] = a.cand_key[at];
      pp[u] = a.cand_pos[at];
    }
  }
  int n = a.row_len[t];
  n = min(max(n, 0), a.n_max);
  const int nch = (n + kTopkChunk - 1) / kTopkChunk;
  auto clear_hist = [&]() {   // lens (the chunk workgroups return the histogram to zero)
    if (threadIdx.x == 0) a.lens[t] = min(n, k);
  };
  if (n <= k) {
    for (int i = n + threadIdx.x; i < k; i += kNT) out[i] = -1;
    clear_hist();
    return;
  }
  const uint32_t d1 = a.thr1[2 * t];
  const uint32_t above1 = a.thr1[2 * t + 1];
  {
    // exclusive prefixes of the per-chunk candidate counts: thread i owns chunks 2i, 2i + 1
    const uint32_t v0 = c0 < nch ? r0 : 0u;
    const uint32_t v1 = c0 + 1 < nch ? r1 : 0u;
    for (int i = threadIdx.x; i < kHistBins; i += kNT) s_hist[i] = 0;
    if (threadIdx.x == 0) s_res[4] = 0;           // set below if a chunk overflows SJ
    // up to 128 chunks every count sits in wave 0 (the other waves hold zeros): a wave scan,
    // no workgroup barriers
    uint32_t total, incl;
    if (nch <= 128) {
      incl = wave_incl_scan(v0 + v1);
      total = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
    } else {
      incl = block_incl_scan<kNT>(v0 + v1, s_w, &total);
    }
    if (c0 < nch) s_off[c0] = incl - v0 - v1;
    if (c0 + 1 < nch) s_off[c0 + 1] = incl - v1;
    if (threadIdx.x == 0) s_off[nch] = total;
    if (sj_log >= 6 && (v0 > (1u << sj_log) || v1 > (1u << sj_log))) s_res[4] = 1;
    lds_barrier();
  }
  const bool spec = sj_log >= 6 && s_res[4] == 0;    // uniform
  const uint32_t n_cand = s_off[nch];
  const bool in_lds = CAND > 0 && n_cand <= (uint32_t)CAND;
  // Chunk of candidate i (candidates are numbered chunk by chunk): the largest c < nch with
  // prefix[c] <= i, by binary lifting with a uniform number of steps, so that several lookups
  // interleave their LDS reads. prefix[nch] = n_cand > i stops every probe past the end.
  const int steps = nch <= 1 ? 0 : 32 - __clz(nch - 1);
  auto cand_at = [&](uint32_t i) -> int64_t {
    int lo = 0;
    for (int r = steps - 1; r >= 0; --r) {
      const int probe = lo + (1 << r);
      if (s_off[min(probe, nch)] <= i) lo = probe;
    }
    return ((int64_t)t * a.n_chunks + lo) * kTopkChunk + (i - s_off[lo]);
  };
  auto key_of = [&](uint32_t i) { return in_lds ? s_ck[i] : a.cand_key[cand_at(i)]; };
  auto pos_of = [&](uint32_t i) { return in_lds ? s_cp[i] : a.cand_pos[cand_at(i)]; };
  // 1. gather the candidates; histogram of their second digit. In registers: slot u of this
  // thread holds a candidate when bit u of vmask is set (the speculative layout above, or
  // candidate u * kNT + thread of the general path).
  const bool in_regs = n_cand <= (uint32_t)(RU * kNT);
  uint32_t vmask = 0;
  if (spec) {
#pragma unroll
    for (int u = 0; u < RU; ++u) {
      const int q = u * kNT + threadIdx.x;
      const int c = q >> sj_log;
      const uint32_t j = (uint32_t)(q & ((1 << sj_log) - 1));
      if (c < nch && j < s_off[c + 1] - s_off[c]) {
        vmask |= 1u << u;
        atomicAdd(&s_hist[(kk[u] >> D2) & (kHistBins - 1)], 1u);
      }
    }
  } else {
#pragma unroll
    for (int u = 0; u < RU; ++u) vmask |= (uint32_t)(u * kNT + threadIdx.x < (int)n_cand) << u;
  }
  for (uint32_t i0 = 0; !spec && i0 < n_cand; i0 += RU * kNT) {
    // lanes past the end re-read the last candidate (n_cand >= 1: the bin holds the k-th key)
    uint32_t ic[RU];
    int lo[RU];
#pragma unroll
    for (int u = 0; u < RU; ++u) {
      ic[u] = min(i0 + u * kNT + threadIdx.x, n_cand - 1);
      lo[u] = 0;
    }
    for (int r = steps - 1; r >= 0; --r) {
#pragma unroll
      for (int u = 0; u < RU; ++u) {
        const int probe = lo[u] + (1 << r);
        if (s_off[min(probe, nch)] <= ic[u]) lo[u] = probe;
      }
    }
#pragma unroll
    for (int u = 0; u < RU; ++u) {
      const int64_t at = ((int64_t)t * a.n_chunks + lo[u]) * kTopkChunk + (ic[u] - s_off[lo[u]]);
      kk[u] = a.cand_key[at];
      pp[u] = a.cand_pos[at];
    }
#pragma unroll
    for (int u = 0; u < RU; ++u) {
      const uint32_t i = i0 + u * kNT + threadIdx.x;
      if (i < n_cand) {
        if (in_lds && !in_regs) { s_ck[i] = kk[u]; s_cp[i] = pp[u]; }
        atomicAdd(&s_hist[(kk[u] >> D2) & (kHistBins - 1)], 1u);
      }
    }
  }
  lds_barrier();
  const uint32_t need1 = (uint32_t)k - above1;
  find_digit_desc<kNT>(s_hist, kHistBins, need1, s_w, s_res);
  const uint32_t pre = (d1 << kHistBits) | s_res[0];     // top 24 bits of the threshold key
  uint32_t need = need1 - s_res[1], eq = 0, pos_thr = 0;
  const uint32_t sub = s_hist[s_res[0]];                  // candidates in the threshold sub-bin
  lds_barrier();
  // 2. the threshold sub-bin: its last 8 bits, then ties toward the smaller position; a
  // sub-bin that holds exactly the candidates still needed (the usual case: a 24-bit prefix
  // rarely holds more than one) is taken whole
  uint32_t thr;
  if (sub == need) {
    thr = pre << D2;
    eq = need;
  } else if (in_regs) {
    auto get_key = [&](int u, uint32_t& key) {
      key = kk[u];
      return (vmask >> u & 1u) != 0;
    };
    thr = radix_select_regs<kNT, RU>(get_key, pre << D2, ~0u << D2, D2, need, &eq, s_hist, s_w, s_res);
    if (eq > need) {
      uint32_t need2 = need, eq2 = 0;
      auto get_tie = [&](int u, uint32_t& key) {
        key = ~(uint32_t)pp[u];
        return (vmask >> u & 1u) != 0 && kk[u] == thr;
      };
      pos_thr = radix_select_regs<kNT, RU>(get_tie, 0u, 0u, 32, need2, &eq2, s_hist, s_w, s_res);
    }
  } else {
    auto get_key = [&](int i, uint32_t& key) { key = key_of((uint32_t)i); return true; };
    thr = radix_select_desc<kNT>((int)n_cand, get_key, pre << D2, ~0u << D2, D2, need, &eq, s_hist, s_w, s_res);
    if (eq > need) {
      uint32_t need2 = need, eq2 = 0;
      auto get_tie = [&](int i, uint32_t& key) {
        key = ~(uint32_t)pos_of((uint32_t)i);
        return key_of((uint32_t)i) == thr;
      };
      pos_thr = radix_select_desc<kNT>((int)n_cand, get_tie, 0u, 0u, 32, need2, &eq2, s_hist, s_w, s_res);
    }
  }
  const bool all_ties = eq <= need;
  auto selected = [&](uint32_t key, int32_t pos) {
    const uint32_t hi = key >> D2;
    return hi > pre || (hi == pre && (key > thr || (key == thr && (all_ties || ~(uint32_t)pos >= pos_thr))));
  };
  // 3. write the selected candidates after the keys above the bin, thread-major (candidate
  // thread + j * kNT for j = 0, 1, ... in both forms)
  uint32_t tot;
  if (in_regs) {
    uint32_t sel = 0, m = 0;
#pragma unroll
    for (int u = 0; u < RU; ++u) {
      const bool x = (vmask >> u & 1u) != 0 && selected(kk[u], pp[u]);
      sel |= (uint32_t)x << u;
      m += x;
    }
    uint32_t o = above1 + block_incl_scan<kNT>(m, s_w, &tot) - m;
#pragma unroll
    for (int u = 0; u < RU; ++u)
      if (sel >> u & 1u) {
        if (o < (uint32_t)k) out[o] = pp[u];
        ++o;
      }
  } else {
    uint32_t m = 0;
    for (uint32_t i = threadIdx.x; i < n_cand; i += kNT) m += selected(key_of(i), pos_of(i));
    uint32_t o = above1 + block_incl_scan<kNT>(m, s_w, &tot) - m;
    for (uint32_t i = threadIdx.x; i < n_cand; i += kNT) {
      const int32_t pos = pos_of(i);
      if (selected(key_of(i), pos)) {
        if (o < (uint32_t)k) out[o] = pos;
        ++o;
      }
    }
  }
  clear_hist();   // last: stores in flight would hold up every wait above (vmcnt counts them)
}

hipError_t launch_topk_lds(const TopkArgs& a, int T, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  // (8704 keeps the causal prefill of 8K tokens plus a few, e.g. the 8193 candidates of its last
  // row, at three workgroups per CU)
  if (a.n_max <= 8704) launch_kernel(k_topk_lds<8704>, dim3(T), dim3(kNT), st, a);
  else launch_kernel(k_topk_lds<kTopkLdsMax>, dim3(T), dim3(kNT), st, a);   // 32 keys a thread
  return hipGetLastError();
}

static int topk_chunks(const TopkArgs& a) { return max(1, (a.n_max + kTopkChunk - 1) / kTopkChunk); }

hipError_t launch_topk_hist(const TopkArgs& a, int T, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  launch_kernel(k_topk_hist, dim3(topk_chunks(a), T), dim3(kNT), st, a);
  return hipGetLastError();
}

hipError_t launch_topk_filter(const TopkArgs& a, int T, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  launch_kernel(k_topk_filter, dim3(topk_chunks(a), T), dim3(kNT), st, a);
  return hipGetLastError();
}

hipError_t launch_topk_finalize(const TopkArgs& a, int T, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  const dim3 grid(a.n_chunks + 1, T);
  if ((int64_t)grid.x * T <= 256) launch_kernel(k_topk_finalize<kTopkCandLds>, grid, dim3(kNT), st, a);
  else launch_kernel(k_topk_finalize<0>, grid, dim3(kNT), st, a);
  return hipGetLastError();
}

}  // namespace dsa
