// Kernel argument blocks and host launchers of the DSA library (internal).
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

#include "common.hpp"

namespace dsa {

// Kernel timing. In the library's timing mode the wrapper around a launch sets these events;
// the launch records them from its own dispatch packet (kernel start and end: the interval a
// kernel-trace profiler reports) and clears them.
struct LaunchEvents {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};
extern thread_local LaunchEvents t_launch_events;

template <class... P, class... A>
inline void launch_kernel(void (*k)(P...), dim3 grid, dim3 block, hipStream_t st, A... args) {
  const LaunchEvents ev = t_launch_events;
  t_launch_events = LaunchEvents{};
  hipExtLaunchKernelGGL(k, grid, block, 0, st, ev.start, ev.stop, 0, args...);
}

// top-k radix: first digit = top 12 bits of the order-preserving key
constexpr int kHistBits = 12;
constexpr int kHistBins = 1 << kHistBits;
// copies of each row's global first-digit histogram, written by alternate workgroups: the
// score kernel's atomics on the few busy bins serialise per address, so more copies shorten
// that tail, at the price of a longer histogram read in every filter workgroup
constexpr int kHistSlices = 2;
// rows with at most this many candidates are selected by one workgroup entirely in LDS
constexpr int kTopkLdsMax = 16384;
// candidates per workgroup in the multi-workgroup (long row) select
constexpr int kTopkChunk = 4096;
// the finalize step keeps the threshold bin's candidates in LDS when there are at most this
// many (else it re-reads them from the workspace)
constexpr int kTopkCandLds = 8192;
// chunks per row (long rows up to kMaxChunks * kTopkChunk = 4M candidates)
constexpr int kMaxChunks = 1024;

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
// many rows sharing keys (prefill): 8 rows per workgroup share each key tile; bf16 keys,
// slots < 2^31
hipError_t launch_index_scores_prefill(const ScoreArgs& a, int di, int T, hipStream_t st);

struct TopkArgs {
  const float* logits;
  int64_t ld_logits;
  const int32_t* row_len;
  int32_t n_max;
  int32_t topk;
  int32_t* indices;
  int64_t ld_idx;
  int32_t* lens;
  // long-row path workspace (per row: n_chunks = ceil(n_max / kTopkChunk) chunk regions)
  uint32_t* hist;          // [T, kHistSlices, kHistBins] first-digit histogram, zero at rest
  uint32_t* thr1;          // [T, 2]: (first digit of the threshold, count above its bin)
  uint32_t* cand_key;      // [T, n_chunks, kTopkChunk] threshold-bin candidates: keys
  int32_t* cand_pos;       // and positions
  uint32_t* counts;        // [T, n_chunks, 2]: (above the bin, in the bin) per chunk
  int32_t n_chunks;
};

hipError_t launch_topk_lds(const TopkArgs& a, int T, hipStream_t st);
hipError_t launch_topk_hist(const TopkArgs& a, int T, hipStream_t st);
hipError_t launch_topk_filter(const TopkArgs& a, int T, hipStream_t st);
hipError_t launch_topk_finalize(const TopkArgs& a, int T, hipStream_t st);

// uniform pools hold OCP e4m3 (kFmtUniform) or fnuz e4m3 (kFmtFnuz) bytes, same layout
enum KvFmt { kFmtBf16 = 0, kFmtUniform = 1, kFmtDsMla = 2, kFmtFnuz = 3 };
template <int FMT>
constexpr bool kUniformFmt = FMT == kFmtUniform || FMT == kFmtFnuz;

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
  int32_t H;               // heads of q, out, lse and sink
  int32_t Hp;              // H rounded up to whole 16-head tiles: the head grid and the partials
  int32_t n_split;         // workgroups per (row, head group)
  int32_t rows_per_split;  // multiple of 32
  float scale_log2;        // softmax_scale * log2(e)
  uint16_t* out;           // bf16 [T, H, 512]
  int64_t ld_out;
  float* lse;              // [T, H] or nullptr
  const float* sink;       // [H] per-head sink logit (natural-log units) or nullptr
  int32_t lse_log2;        // lse in base 2 instead of natural log
  float* part_o;           // [T, Hp, n_split, 512]
  float* part_ml;          // [T, Hp, n_split, 2]
};

hipError_t launch_sparse_mla(const MlaArgs& a, int fmt, int d_qk, int ht, int nbuf, int T, hipStream_t st);
hipError_t launch_mla_combine(const MlaArgs& a, int T, hipStream_t st);

// backward of the sparse MLA attention: one list, bf16 rows
struct MlaBwdArgs {
  const uint16_t* q;       // bf16 [T, H, d_qk]
  int64_t ld_q;
  KvDev kv;
  const int32_t* idx;      // [T, n_idx]
  int64_t ld_idx;
  int32_t n_idx;
  const int32_t* row_req;  // nullptr: row t is request t
  int32_t n_req;
  int32_t H;               // heads of q, out, lse, dout, dq and sink
  int32_t Hp;              // 16, 32, 64 or 128 >= H: the head grid and the workspace rows
  float scale;             // softmax_scale
  float scale_log2;        // softmax_scale * log2(e)
  const uint16_t* out;     // bf16 [T, H, 512] (the forward's output)
  int64_t ld_out;
  const float* lse;        // [T, H] the forward's lse
  int32_t lse_log2;        // lse in base 2
  const uint16_t* dout;    // bf16 [T, H, 512]
  int64_t ld_dout;
  const float* sink;       // [H] or nullptr
  float* dq;               // fp32 [T, H, d_qk]
  int64_t ld_dq;
  float* dkv;              // fp32 [n_slots, d_qk], added to
  float* dsink;            // fp32 [H], added to, or nullptr
  uint16_t* ws_dz;         // workspace: bf16 [T, n_idx, Hp] softmax_scale * dZ
  uint16_t* ws_p;          // workspace: bf16 [T, n_idx, Hp] P
  int32_t* ws_slot;        // workspace: [T, n_idx] slots (-1: padding)
  int32_t* ws_owner;       // workspace: [n_slots] who lists each slot (nullptr: atomics only)
  int64_t n_slots;         // the cache's slot count (with ws_owner)
  float* ws_dqp;           // workspace: [nsplit - 1, T, H, d_qk] dq of list parts 1..nsplit-1
  int32_t nsplit;          // parts each row's list is split into (first kernel's grid z)
};

// parts of each row's list in the backward's first kernel: enough workgroups (two 16-head
// groups each) for about one per CU, every part at least 8 blocks of 32 entries
int bwd_splits(int T, int Hp, int n_idx);

hipError_t launch_sparse_mla_bwd(const MlaBwdArgs& a, int d_qk, int T, hipStream_t st);
hipError_t launch_sparse_mla_bwd_mid(const MlaBwdArgs& a, int d_qk, int T, hipStream_t st);
hipError_t launch_sparse_mla_bwd_dkv(const MlaBwdArgs& a, int d_qk, int T, hipStream_t st);

// cache writes: bf16 rows -> a cache format, one row per token at slots[token]
enum { kCwBf16 = 0, kCwScaled = 1, kCwDsMla = 2, kCwScaledFnuz = 3 };
struct CacheWriteArgs {
  const uint16_t* src;     // bf16 [n_tok, ld_src]
  int64_t ld_src;
  int32_t n_tok;
  int32_t D;               // channels per row
  const int32_t* slots;    // [n_tok]; -1 or out of range: skipped
  int64_t n_slots;
  uint8_t* data;           // cache bytes (layout per kind)
  float* fscale;           // kCwScaled(Fnuz): [n_slots, D / group]
  int32_t group;           // kCwScaled(Fnuz): channels per fp32 scale
  int32_t page;            // kCwDsMla: tokens per page
};
hipError_t launch_cache_write(const CacheWriteArgs& a, int kind, hipStream_t st);

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t st);

}  // namespace dsa
