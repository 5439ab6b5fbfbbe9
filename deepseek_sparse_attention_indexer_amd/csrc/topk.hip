// Per-row top-k of the indexer scores on gfx950.
//
// Output contract (decode top-k wrapper of tokenspeed PR 627 "Add gluon kernel for DSA",
// review: it returns (out, lens_out)): indices[t, 0:topk] hold the positions of the
// min(topk, n_t) largest scores in unspecified order, then -1; lens[t] = min(topk, n_t).
// Ties are broken toward the smaller position, so the selected SET is deterministic.
//
// Method: radix select on the order-preserving uint32 image of the fp32 scores, most
// significant digit first, counting with histograms and reserving output slots with atomic
// adds (the threshold / greater / equal counting of the PR 627 selector). Digits are 12, 12
// and 8 bits. When more candidates share the threshold key than slots remain, the ties are
// resolved by a second radix select on the complemented position.
//
//  * k_topk_lds: one 512-thread workgroup per row, the row's keys held in LDS (<= 16K).
//  * long rows: the first-digit histogram is built per chunk (k_topk_hist, or fused into
//    the score kernel), k_topk_filter's workgroups each emit their chunk's candidates above
//    the threshold bin and append the threshold bin's candidates to a list, and the last
//    workgroup to finish (atomic ticket) resolves that list exactly and clears the row's
//    control words and histogram for the next call.
#include "common.hpp"
#include "kernels.hpp"

namespace dsa {

constexpr int kNT = 512;   // threads of the select workgroups

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    uint32_t u = __shfl_up(v, d);
    if (lane >= d) v += u;
  }
  return v;
}

// Inclusive scan over the workgroup (thread order). s_w: kNT/64 words of LDS.
__device__ __forceinline__ uint32_t block_incl_scan(uint32_t v, uint32_t* s_w, uint32_t* total) {
  constexpr int NW = kNT / 64;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const uint32_t x = wave_incl_scan(v);
  __syncthreads();
  if (lane == 63) s_w[w] = x;
  __syncthreads();
  uint32_t off = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const uint32_t y = s_w[i];
    off += (i < w) ? y : 0u;
    tot += y;
  }
  if (total) *total = tot;
  return x + off;
}

// Digit d (0..nb-1) of a histogram such that (count of digits > d) < need <= (count >= d).
// Writes s_res[0] = d, s_res[1] = count of digits > d. Requires sum(h) >= need >= 1.
__device__ void find_digit_desc(const uint32_t* h, int nb, uint32_t need, uint32_t* s_w,
                                uint32_t* s_res) {
  const int per = nb >= kNT ? nb / kNT : 1;
  const int act = nb / per;
  const int tid = threadIdx.x;
  uint32_t local = 0;
  if (tid < act)
    for (int i = 0; i < per; ++i) local += h[nb - 1 - (tid * per + i)];
  const uint32_t incl = block_incl_scan(local, s_w, nullptr);
  const uint32_t excl = incl - local;
  if (tid < act && excl < need && need <= incl) {
    uint32_t acc = excl;
    for (int i = 0; i < per; ++i) {
      const int bin = nb - 1 - (tid * per + i);
      const uint32_t cnt = h[bin];
      if (acc + cnt >= need) {
        s_res[0] = (uint32_t)bin;
        s_res[1] = acc;
        break;
      }
      acc += cnt;
    }
  }
  __syncthreads();
}

// Radix select (descending) over items i < cnt for which get(i, key) is true and whose key
// matches `prefix` under `pmask`. Resolves the low `low_bits` bits in 12-bit digits; on
// return `need` is the number still to take among keys equal to the returned threshold and
// *eq_count the number of such keys.
template <class Get>
__device__ uint32_t radix_select_desc(int cnt, Get get, uint32_t prefix, uint32_t pmask,
                                      int low_bits, uint32_t& need, uint32_t* eq_count,
                                      uint32_t* s_hist, uint32_t* s_w, uint32_t* s_res) {
  int shift = low_bits;
  uint32_t last_eq = 0;
  while (shift > 0) {
    const int bits = shift >= 12 ? 12 : shift;
    shift -= bits;
    const int nb = 1 << bits;
    const uint32_t dm = (uint32_t)(nb - 1);
    for (int i = threadIdx.x; i < nb; i += kNT) s_hist[i] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < cnt; i += kNT) {
      uint32_t key;
      if (get(i, key) && (key & pmask) == prefix) atomicAdd(&s_hist[(key >> shift) & dm], 1u);
    }
    __syncthreads();
    find_digit_desc(s_hist, nb, need, s_w, s_res);
    const uint32_t d = s_res[0];
    need -= s_res[1];
    last_eq = s_hist[d];
    prefix |= d << shift;
    pmask |= dm << shift;
    __syncthreads();
  }
  *eq_count = last_eq;
  return prefix;
}

// ------------------------------------------------------------------ rows that fit in LDS
__global__ __launch_bounds__(kNT) void k_topk_lds(TopkArgs a) {
  __shared__ uint32_t s_key[kTopkLdsMax];
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
  for (int i = threadIdx.x; i < n; i += kNT) s_key[i] = float_key(row[i]);
  if (threadIdx.x == 0) s_res[2] = 0;
  __syncthreads();

  uint32_t need = (uint32_t)k, eq = 0;
  auto get_key = [&](int i, uint32_t& key) { key = s_key[i]; return true; };
  const uint32_t thr = radix_select_desc(n, get_key, 0u, 0u, 32, need, &eq, s_hist, s_w, s_res);
  // ties at thr: keep the `need` smallest positions (largest complemented positions)
  uint32_t pos_thr = 0u;
  if (eq > need) {
    uint32_t need2 = need, eq2 = 0;
    auto get_tie = [&](int i, uint32_t& key) { key = ~(uint32_t)i; return s_key[i] == thr; };
    pos_thr = radix_select_desc(n, get_tie, 0u, 0u, 32, need2, &eq2, s_hist, s_w, s_res);
  }
  const bool all_ties = eq <= need;
  for (int i = threadIdx.x; i < n; i += kNT) {
    const uint32_t key = s_key[i];
    const bool sel = key > thr || (key == thr && (all_ties || ~(uint32_t)i >= pos_thr));
    if (sel) {
      const uint32_t o = atomicAdd(&s_res[2], 1u);
      if (o < (uint32_t)k) out[o] = i;
    }
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
  for (int i = threadIdx.x; i < kHistBins; i += kNT) s_hist[i] = 0;
  __syncthreads();
  const float* row = a.logits + (int64_t)t * a.ld_logits;
  const int s1 = min(n, s0 + kTopkChunk);
  for (int s = s0 + threadIdx.x; s < s1; s += kNT)
    atomicAdd(&s_hist[float_key(row[s]) >> (32 - kHistBits)], 1u);
  __syncthreads();
  uint32_t* gh = a.hist + ((int64_t)t * kHistSlices + (blockIdx.x % kHistSlices)) * kHistBins;
  for (int i = threadIdx.x; i < kHistBins; i += kNT) {
    const uint32_t v = s_hist[i];
    if (v) atomicAdd(gh + i, v);
  }
}

__global__ __launch_bounds__(kNT) void k_topk_filter(TopkArgs a) {
  __shared__ uint32_t s_hist[kHistBins];
  __shared__ uint32_t s_w[kNT / 64];
  __shared__ uint32_t s_res[8];

  const int t = blockIdx.y;
  const int k = a.topk;
  int n = a.row_len[t];
  n = min(max(n, 0), a.n_max);
  int32_t* out = a.indices + (int64_t)t * a.ld_idx;
  TopkCtl* ctl = a.ctl + t;
  uint32_t* gh = a.hist + (int64_t)t * kHistSlices * kHistBins;
  const float* row = a.logits + (int64_t)t * a.ld_logits;
  const int s0 = blockIdx.x * kTopkChunk;
  const int s1 = min(n, s0 + kTopkChunk);
  const int per = kTopkChunk / kNT;

  uint32_t d1 = 0, above1 = 0;
  if (n <= k) {
    for (int s = s0 + threadIdx.x; s < s1; s += kNT) out[s] = s;
  } else {
    // first digit of the threshold from the row's histogram
    for (int i = threadIdx.x; i < kHistBins; i += kNT) {
      uint32_t v = 0;
#pragma unroll
      for (int sl = 0; sl < kHistSlices; ++sl) v += gh[sl * kHistBins + i];
      s_hist[i] = v;
    }
    __syncthreads();
    find_digit_desc(s_hist, kHistBins, (uint32_t)k, s_w, s_res);
    d1 = s_res[0];
    above1 = s_res[1];
    // this chunk: emit keys above the threshold bin, append the threshold bin to the list
    uint32_t keys[kTopkChunk / kNT];
    uint32_t n_gt = 0, n_eq = 0;
#pragma unroll
    for (int j = 0; j < per; ++j) {
      const int s = s0 + j * kNT + threadIdx.x;
      uint32_t key = 0;
      if (s < s1) {
        key = float_key(row[s]);
        const uint32_t dg = key >> (32 - kHistBits);
        n_gt += dg > d1;
        n_eq += dg == d1;
      }
      keys[j] = key;
    }
    uint32_t tot_gt, tot_eq;
    const uint32_t inc_gt = block_incl_scan(n_gt, s_w, &tot_gt);
    __syncthreads();
    const uint32_t inc_eq = block_incl_scan(n_eq, s_w, &tot_eq);
    if (threadIdx.x == 0) {
      s_res[4] = tot_gt ? atomicAdd(&ctl->sel, tot_gt) : 0u;
      s_res[5] = tot_eq ? atomicAdd(&ctl->cand, tot_eq) : 0u;
    }
    __syncthreads();
    uint32_t o_gt = s_res[4] + inc_gt - n_gt;
    uint32_t o_eq = s_res[5] + inc_eq - n_eq;
    uint32_t* ck = a.cand_key + (int64_t)t * a.n_max;
    int32_t* cp = a.cand_pos + (int64_t)t * a.n_max;
#pragma unroll
    for (int j = 0; j < per; ++j) {
      const int s = s0 + j * kNT + threadIdx.x;
      if (s < s1) {
        const uint32_t dg = keys[j] >> (32 - kHistBits);
        // the guards only matter if the histogram disagrees with the scores (a caller that
        // skipped dsa_workspace_init); they keep every store inside the row's buffers
        if (dg > d1) { if (o_gt < (uint32_t)k) out[o_gt] = s; ++o_gt; }
        else if (dg == d1) { if (o_eq < (uint32_t)a.n_max) { ck[o_eq] = keys[j]; cp[o_eq] = s; } ++o_eq; }
      }
    }
  }

  // last workgroup of the row resolves the threshold bin
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) s_res[6] = (atomicAdd(&ctl->done, 1u) == gridDim.x - 1) ? 1u : 0u;
  __syncthreads();
  if (!s_res[6]) return;
  __threadfence();

  if (n <= k) {
    for (int i = n + threadIdx.x; i < k; i += kNT) out[i] = -1;
  } else {
    const int cnt = min((int)__hip_atomic_load(&ctl->cand, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT), a.n_max);
    const uint32_t* ck = a.cand_key + (int64_t)t * a.n_max;
    const int32_t* cp = a.cand_pos + (int64_t)t * a.n_max;
    uint32_t need = (uint32_t)k - above1, eq = 0;
    auto get_key = [&](int i, uint32_t& key) { key = ck[i]; return true; };
    const uint32_t hi_mask = ~0u << (32 - kHistBits);
    const uint32_t thr = radix_select_desc(cnt, get_key, d1 << (32 - kHistBits), hi_mask,
                                           32 - kHistBits, need, &eq, s_hist, s_w, s_res);
    uint32_t pos_thr = 0u;
    if (eq > need) {
      uint32_t need2 = need, eq2 = 0;
      auto get_tie = [&](int i, uint32_t& key) { key = ~(uint32_t)cp[i]; return ck[i] == thr; };
      pos_thr = radix_select_desc(cnt, get_tie, 0u, 0u, 32, need2, &eq2, s_hist, s_w, s_res);
    }
    const bool all_ties = eq <= need;
    if (threadIdx.x == 0) s_res[7] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < cnt; i += kNT) {
      const uint32_t key = ck[i];
      const bool sel = key > thr || (key == thr && (all_ties || ~(uint32_t)cp[i] >= pos_thr));
      if (sel) {
        const uint32_t o = above1 + atomicAdd(&s_res[7], 1u);
        if (o < (uint32_t)k) out[o] = cp[i];
      }
    }
  }
  for (int i = threadIdx.x; i < kHistSlices * kHistBins; i += kNT) gh[i] = 0;
  if (threadIdx.x == 0) {
    a.lens[t] = min(n, k);
    ctl->sel = 0;
    ctl->cand = 0;
    ctl->done = 0;
  }
}

hipError_t launch_topk_lds(const TopkArgs& a, int T, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_topk_lds, dim3(T), dim3(kNT), 0, st, a);
  return hipGetLastError();
}

static int topk_chunks(const TopkArgs& a) { return max(1, (a.n_max + kTopkChunk - 1) / kTopkChunk); }

hipError_t launch_topk_hist(const TopkArgs& a, int T, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_topk_hist, dim3(topk_chunks(a), T), dim3(kNT), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_topk_filter(const TopkArgs& a, int T, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_topk_filter, dim3(topk_chunks(a), T), dim3(kNT), 0, st, a);
  return hipGetLastError();
}

}  // namespace dsa
