// Kernel argument blocks and host launchers of the DSA library (internal).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace dsa {

// top-k radix: first digit = top 12 bits of the order-preserving key
constexpr int kHistBits = 12;
constexpr int kHistBins = 1 << kHistBits;
// copies of each row's global first-digit histogram, spread over workgroups to thin out
// same-address atomics
constexpr int kHistSlices = 4;
// rows with at most this many candidates are selected by one workgroup entirely in LDS
constexpr int kTopkLdsMax = 16384;
// candidates per workgroup in the multi-workgroup (long row) select
constexpr int kTopkChunk = 4096;

struct ScoreArgs {
  const uint16_t* q_idx;   // bf16 [T, Hi, di]
  int64_t ld_q;
  const float* w;          // [T, Hi]
  int64_t ld_w;
  const void* keys;        // bf16 or fp8 [slots, di]
  const float* key_scale;  // fp8: [slots]
  Paging pg;
  const int32_t* row_req;
  const int32_t* row_len;
  int32_t n_max;
  int32_t Hi;
  float index_scale;
  int32_t n_req;           // requests (rows of the page table / req_base)
  float* logits;
  int64_t ld_logits;
  uint32_t* hist;          // [T, kHistSlices, kHistBins] or nullptr
};

hipError_t launch_index_scores(const ScoreArgs& a, int di, bool fp8, bool hist, int T,
                               hipStream_t st);

// Per-row control words of the long-row select (zero at rest).
struct TopkCtl {
  uint32_t sel;     // selected so far (first-digit bins above the threshold bin)
  uint32_t cand;    // candidates in the threshold bin
  uint32_t done;    // finished workgroups
  uint32_t _pad;
};

struct TopkArgs {
  const float* logits;
  int64_t ld_logits;
  const int32_t* row_len;
  int32_t n_max;
  int32_t topk;
  int32_t* indices;
  int64_t ld_idx;
  int32_t* lens;
  // long-row path workspace
  TopkCtl* ctl;            // [T]
  uint32_t* hist;          // [T, kHistSlices, kHistBins]
  uint32_t* cand_key;      // [T, n_max]
  int32_t* cand_pos;       // [T, n_max]
};

hipError_t launch_topk_lds(const TopkArgs& a, int T, hipStream_t st);
hipError_t launch_topk_hist(const TopkArgs& a, int T, hipStream_t st);
hipError_t launch_topk_filter(const TopkArgs& a, int T, hipStream_t st);

enum KvFmt { kFmtBf16 = 0, kFmtUniform = 1, kFmtDsMla = 2 };

struct KvDev {
  const uint8_t* data;
  const float* scales;     // uniform: [slots, D/64]
  Paging pg;
};

struct MlaArgs {
  const uint16_t* q;       // bf16 [T, H, d_qk]
  int64_t ld_q;
  KvDev kv[2];             // main, extra
  const int32_t* idx[2];
  int64_t ld_idx[2];
  int32_t n_idx[2];
  const int32_t* row_req;  // nullptr: row t is request t
  int32_t n_req;
  int32_t H;
  int32_t n_split;         // workgroups per (row, head group)
  int32_t rows_per_split;  // multiple of 32
  float scale_log2;        // softmax_scale * log2(e)
  uint16_t* out;           // bf16 [T, H, 512]
  int64_t ld_out;
  float* lse;              // [T, H] or nullptr
  float* part_o;           // [T, H, n_split, 512]
  float* part_ml;          // [T, H, n_split, 2]
  uint32_t* counters;      // [T, H / (16 * HT)]
};

hipError_t launch_sparse_mla(const MlaArgs& a, int fmt, int d_qk, int ht, int T, hipStream_t st);

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t st);

}  // namespace dsa
