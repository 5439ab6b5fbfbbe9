// Workgroup-wide selection helpers (gfx950): wave and block scans, the digit of a descending
// radix select, and radix selects over items in LDS, memory or registers. NT = threads of the
// calling workgroup (a multiple of 64). Shared by the top-k kernels and the attention kernel
// that resolves a row's top-k from its threshold-bin candidates.
#pragma once
#include "common.hpp"

namespace dsa {

// Inclusive scan over the 64 lanes with DPP moves (a few cycles each) instead of LDS
// permutes: shifts by 1, 2, 4, 8 inside each row of 16 lanes, then the row totals carried
// forward with the row broadcasts of lane 15 (into rows 1 and 3) and lane 31 (rows 2, 3).
// Lanes without a source read 0 (bound_ctrl).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, true);   // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, true);   // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, true);   // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, true);   // row_shr:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return v;
}

// Inclusive scan over the workgroup of NT threads (thread order). s_w: NT/64 words of LDS.
template <int NT>
__device__ __forceinline__ uint32_t block_incl_scan(uint32_t v, uint32_t* s_w, uint32_t* total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const uint32_t x = wave_incl_scan(v);
  lds_barrier();
  if (lane == 63) s_w[w] = x;
  lds_barrier();
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
template <int NT>
__device__ void find_digit_desc(const uint32_t* h, int nb, uint32_t need, uint32_t* s_w,
                                uint32_t* s_res) {
  const int per = nb >= NT ? nb / NT : 1;
  const int act = nb / per;
  const int tid = threadIdx.x;
  uint32_t local = 0;
  if (tid < act)
    for (int i = 0; i < per; ++i) local += h[nb - 1 - (tid * per + i)];
  const uint32_t incl = block_incl_scan<NT>(local, s_w, nullptr);
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
  lds_barrier();
}

// Radix select (descending) over items i < cnt for which get(i, key) is true and whose key
// matches `prefix` under `pmask`. Resolves the low `low_bits` bits in 12-bit digits; on
// return `need` is the number still to take among keys equal to the returned threshold and
// *eq_count the number of such keys. It stops early once the threshold digit's bin holds
// exactly the keys still needed: every key with that prefix is taken, so the remaining low
// bits of the returned threshold are zero and *eq_count == need (a caller that takes the keys
// above the threshold and, when *eq_count <= need, all keys equal to it selects exactly them).
template <int NT, class Get>
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
    for (int i = threadIdx.x; i < nb; i += NT) s_hist[i] = 0;
    lds_barrier();
    for (int i = threadIdx.x; i < cnt; i += NT) {
      uint32_t key;
      if (get(i, key) && (key & pmask) == prefix) atomicAdd(&s_hist[(key >> shift) & dm], 1u);
    }
    lds_barrier();
    find_digit_desc<NT>(s_hist, nb, need, s_w, s_res);
    const uint32_t d = s_res[0];
    need -= s_res[1];
    last_eq = s_hist[d];
    prefix |= d << shift;
    pmask |= dm << shift;
    lds_barrier();
    if (last_eq == need) break;   // uniform: the bin is taken whole
  }
  *eq_count = last_eq;
  return prefix;
}

// The same radix select over items held in registers: item u (< U) of every thread, taken
// when get(u, key) is true.
template <int NT, int U, class Get>
__device__ uint32_t radix_select_regs(Get get, uint32_t prefix, uint32_t pmask, int low_bits,
                                      uint32_t& need, uint32_t* eq_count, uint32_t* s_hist,
                                      uint32_t* s_w, uint32_t* s_res) {
  int shift = low_bits;
  uint32_t last_eq = 0;
  while (shift > 0) {
    const int bits = shift >= 12 ? 12 : shift;
    shift -= bits;
    const int nb = 1 << bits;
    const uint32_t dm = (uint32_t)(nb - 1);
    for (int i = threadIdx.x; i < nb; i += NT) s_hist[i] = 0;
    lds_barrier();
#pragma unroll
    for (int u = 0; u < U; ++u) {
      uint32_t key;
      if (get(u, key) && (key & pmask) == prefix) atomicAdd(&s_hist[(key >> shift) & dm], 1u);
    }
    lds_barrier();
    find_digit_desc<NT>(s_hist, nb, need, s_w, s_res);
    const uint32_t d = s_res[0];
    need -= s_res[1];
    last_eq = s_hist[d];
    prefix |= d << shift;
    pmask |= dm << shift;
    lds_barrier();
    if (last_eq == need) break;   // uniform: the bin is taken whole
  }
  *eq_count = last_eq;
  return prefix;
}

}  // namespace dsa
