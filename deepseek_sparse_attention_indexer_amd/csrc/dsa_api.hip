// C ABI of the DSA layer hot path: argument checks, workspace carving, launch policies.
// See include/dsa.h for the contract of every entry point.
#include <math.h>
#include <algorithm>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include <mutex>
#include <vector>

#include "dsa.h"
#include "kernels.hpp"

namespace dsa {
thread_local LaunchEvents t_launch_events;
}  // namespace dsa

using namespace dsa;

namespace {

// ---------------------------------------------------------------- workspace layout
// Header of control words that are zero at rest (every entry restores them before its last
// kernel ends). It has a fixed size, so data regions of one problem never overlap control
// words of another and one workspace can serve every entry and problem size.
constexpr int kMaxLongRows = 64;                  // long-row top-k rows per launch batch
constexpr int kPrefillMinRows = 64;               // rows from which the shared-key score kernel is used
constexpr int64_t align256(int64_t v) { return (v + 255) & ~int64_t(255); }
constexpr int64_t kOffHist = 0;
constexpr int64_t kHeaderBytes = align256(kOffHist + (int64_t)kMaxLongRows * kHistSlices * kHistBins * 4);

struct Carve {
  int64_t off = kHeaderBytes;
  int64_t take(int64_t bytes) {
    const int64_t o = off;
    off = align256(off + bytes);
    return o;
  }
};

bool al16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool al4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

int log2_exact(int v) {
  if (v <= 0 || (v & (v - 1))) return -1;
  int s = 0;
  while ((1 << s) < v) ++s;
  return s;
}

dsa_status check_paging(const dsa_paging& p, int64_t n_slots) {
  if (p.page_size < 1 || n_slots < 1) return DSA_ERR_ARG;
  if (p.block_table) {
    if (p.bt_stride < 1 || n_slots % p.page_size) return DSA_ERR_ARG;
    if (n_slots / p.page_size > INT32_MAX) return DSA_ERR_UNSUPPORTED;
  } else if (!p.req_base) {
    return DSA_ERR_ARG;
  }
  return DSA_OK;
}

Paging make_paging(const dsa_paging& p, int64_t n_slots) {
  Paging g;
  g.bt = p.block_table;
  g.req_base = p.req_base;
  g.bt_stride = p.bt_stride;
  g.n_slots = n_slots;
  g.page = p.page_size;
  g.page_shift = log2_exact(p.page_size);
  g.n_pages = (int32_t)(n_slots / p.page_size);
  g._pad = 0;
  return g;
}

dsa_status check_rows(const dsa_rows* r) {
  if (!r || r->T < 0 || r->n_max < 0) return DSA_ERR_ARG;
  if (r->T > 0 && (!r->row_len || r->n_req < 1)) return DSA_ERR_ARG;
  if (r->T > 0 && !r->row_req && r->T > r->n_req) return DSA_ERR_ARG;  // row t is request t
  if (r->T > 65535) return DSA_ERR_UNSUPPORTED;   // grid y/z limit of the row axis
  return DSA_OK;
}

dsa_status hip_status(hipError_t e) { return e == hipSuccess ? DSA_OK : DSA_ERR_HIP; }

// ---------------------------------------------------------------- kernel timing
struct ProfRec {
  const char* name;
  hipEvent_t a, b;
};
bool g_prof = false;
std::vector<ProfRec> g_recs;
std::vector<hipEvent_t> g_event_pool;

hipEvent_t pool_event() {
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// ---------------------------------------------------------------- launch log
// With DSA_LOG set (to anything but "" or "0"; read once per process) every kernel launch
// prints one line on stderr: the kernel and the launch row that chose it (the problem's shape
// and the plan taken for it), set by each driver before its launches.
bool log_on() {
  static const bool on = [] {
    const char* e = getenv("DSA_LOG");
    return e != nullptr && e[0] != 0 && strcmp(e, "0") != 0;
  }();
  return on;
}
thread_local char t_row[320] = "";
void set_row(const char* fmt, ...) {
  if (!log_on()) return;
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(t_row, sizeof(t_row), fmt, ap);
  va_end(ap);
}

// Run one kernel launch; in timing mode the launch records a pair of events at its kernel's
// start and end (launch_kernel), on the stream it runs on.
template <class F>
hipError_t timed(const char* name, hipStream_t st, F&& launch) {
  if (log_on()) fprintf(stderr, "[dsa] %-22s stream %p  %s\n", name, (void*)st, t_row);
  if (!g_prof) return launch();
  ProfRec r{name, pool_event(), pool_event()};
  if (!r.a || !r.b) return launch();
  t_launch_events = LaunchEvents{r.a, r.b};
  const hipError_t e = launch();
  const bool launched = t_launch_events.start == nullptr;
  t_launch_events = LaunchEvents{};
  if (launched && e == hipSuccess) {
    g_recs.push_back(r);
  } else {
    g_event_pool.push_back(r.a);
    g_event_pool.push_back(r.b);
  }
  return e;
}

// ---------------------------------------------------------------- attention policy
// Heads padded to whole 16-head tiles (the forward's workgroups and split partials), and the
// backward's padded count (its dKV kernel sums heads in groups of 16, 32, 64 or 128).
int heads_padded(int H) { return (H + 15) / 16 * 16; }
int heads_padded_bwd(int H) { return H <= 16 ? 16 : H <= 32 ? 32 : H <= 64 ? 64 : 128; }

struct MlaPlan {
  int ht;          // head tiles per workgroup
  int nbuf;        // depth of the block ring in LDS
  int n_split;
  int rows_per_split;
};

// dsa_launch_override: 0 = the table's choice
int g_force_ht = 0;
int g_force_split = 0;

MlaPlan plan_mla(int T, int H, int ntot, bool decode) {
  // A CU sustains only ~25 GB/s of gathers and a lone wave far less, so a decode step with
  // few rows spreads rows AND partial outputs over every CU: one 16-head tile per 4-wave
  // workgroup (the waves split the value columns) and about two workgroups per CU, so two
  // gathered blocks are in flight per CU (splits never go below one 32-row block). With many
  // rows (16 or more) there is enough parallelism to share each gathered block among 64
  // heads instead (a quarter of the gathers; 8-wave workgroups, one per CU), splits only to
  // reach one workgroup per CU. Prefill rows have no split; all heads of a row share each
  // block.
  // Blocks stream through a ring of two.
  MlaPlan p;
  const int tiles = heads_padded(H) / 16;
  const int nblk = std::max(1, (ntot + 31) / 32);
  int s = 1;
  if (decode && !(T >= 16 && tiles % 4 == 0)) {
    p.ht = 1;
    const int64_t base = (int64_t)T * tiles;
    s = (int)std::min<int64_t>((512 + base - 1) / base, nblk);   // about two workgroups per CU
  } else {
    p.ht = tiles % 4 == 0 ? 4 : (tiles % 2 == 0 ? 2 : 1);
    if (decode) {
      const int64_t base = (int64_t)T * (tiles / p.ht);
      s = (int)std::min<int64_t>((256 + base - 1) / base, nblk);  // about one workgroup per CU
    }
  }
  if (g_force_ht > 0) p.ht = g_force_ht;        // validated against the heads by the callers
  if (g_force_split > 0 && decode) s = std::min(g_force_split, nblk);
  s = std::max(1, s);
  const int bps = (nblk + s - 1) / s;           // blocks per split
  p.rows_per_split = bps * 32;
  p.n_split = (nblk + bps - 1) / bps;
  p.nbuf = 2;
  return p;
}

// an overridden head-tile count that does not divide the padded tiles has no kernel
bool plan_ok(int H, const MlaPlan& p) { return (heads_padded(H) / 16) % p.ht == 0; }

void set_mla_row(int T, int H, int n_main, int n_extra, int fmt, int d_qk, bool decode, const MlaPlan& p) {
  set_row("T=%d H=%d (padded %d) list %d+%d fmt=%d d_qk=%d %s: %d head tile(s) of 16 per workgroup, "
          "%d split(s) of %d rows, ring of %d",
          T, H, heads_padded(H), n_main, n_extra, fmt, d_qk, decode ? "decode" : "prefill", p.ht, p.n_split,
          p.rows_per_split, p.nbuf);
}

// backward: bf16 scale * dZ and P per (row, listed entry, padded head), and the entries' slots
int64_t mla_bwd_ws_bytes(int T, int H, int n_idx) {
  const int64_t e = (int64_t)T * n_idx;
  const int hp = heads_padded_bwd(H);
  const int ns = bwd_splits(T, hp, n_idx);
  // dZ and P, the slots, and the dq partial sums of list parts 1.. (sized at d_qk = 576)
  return align256(e * hp * 2) * 2 + align256(e * 4) + (ns > 1 ? align256((int64_t)(ns - 1) * T * hp * 576 * 4) : 0);
}

// the backward's owner map: one int32 per cache slot, in whole 16-byte words
int64_t mla_bwd_owner_bytes(int64_t n_slots) { return align256((n_slots + 3) / 4 * 16); }

int64_t mla_ws_bytes(int T, int H, int ntot, bool decode) {
  const MlaPlan p = plan_mla(T, H, ntot, decode);
  if (p.n_split <= 1) return 0;
  const int64_t hp = heads_padded(H);
  return align256((int64_t)T * hp * p.n_split * 512 * 4) + align256((int64_t)T * hp * p.n_split * 8);
}

int topk_chunks_of(int n_max) { return std::max(1, (n_max + kTopkChunk - 1) / kTopkChunk); }

int64_t topk_ws_bytes(int T, int n_max) {
  if (n_max <= kTopkLdsMax) return 0;
  const int64_t rows = std::min(T, kMaxLongRows);
  const int64_t per = rows * topk_chunks_of(n_max) * (int64_t)kTopkChunk * 4;
  return 2 * align256(per) + align256(rows * topk_chunks_of(n_max) * 8) + align256(rows * 8);
}

// carve the long-row top-k data regions (after the header) and the header's histograms
void carve_topk(TopkArgs& a, Carve& cv, uint8_t* w, int T, int n_max) {
  const int64_t rows = std::min(T, kMaxLongRows);
  a.n_chunks = topk_chunks_of(n_max);
  const int64_t per = rows * a.n_chunks * (int64_t)kTopkChunk * 4;
  a.cand_key = reinterpret_cast<uint32_t*>(w + cv.take(per));
  a.cand_pos = reinterpret_cast<int32_t*>(w + cv.take(per));
  a.counts = reinterpret_cast<uint32_t*>(w + cv.take(rows * a.n_chunks * 8));
  a.thr1 = reinterpret_cast<uint32_t*>(w + cv.take(rows * 8));
  a.hist = reinterpret_cast<uint32_t*>(w + kOffHist);
}

int logits_ld(int n_max) { return ((max(n_max, 1) + 63) / 64) * 64; }

dsa_status check_kv(const dsa_kv_cache* kv, int d_qk) {
  if (!kv || !kv->data || !al16(kv->data)) return DSA_ERR_ARG;
  dsa_status s = check_paging(kv->paging, kv->n_slots);
  if (s != DSA_OK) return s;
  if (kv->n_slots > (int64_t(1) << 30)) return DSA_ERR_UNSUPPORTED;   // slots travel in 30 bits
  if (kv->d_nope + kv->d_rope != d_qk) return DSA_ERR_ARG;
  switch (kv->format) {
    case DSA_KV_BF16:
      if (d_qk != 576 && d_qk != 512) return DSA_ERR_UNSUPPORTED;
      break;
    case DSA_KV_FP8_UNIFORM:
    case DSA_KV_FP8_UNIFORM_FNUZ:
      if (!kv->scales || !al4(kv->scales)) return DSA_ERR_ARG;
      if (d_qk != 576 && d_qk != 512) return DSA_ERR_UNSUPPORTED;
      break;
    case DSA_KV_FP8_DS_MLA:
      if (kv->d_nope != 448 || kv->d_rope != 64) return DSA_ERR_UNSUPPORTED;
      if (!kv->paging.block_table && kv->n_slots % kv->paging.page_size) return DSA_ERR_ARG;
      break;
    default:
      return DSA_ERR_UNSUPPORTED;
  }
  return DSA_OK;
}

int kv_fmt(const dsa_kv_cache* kv) {
  switch (kv->format) {
    case DSA_KV_BF16: return kFmtBf16;
    case DSA_KV_FP8_UNIFORM: return kFmtUniform;
    case DSA_KV_FP8_UNIFORM_FNUZ: return kFmtFnuz;
    default: return kFmtDsMla;
  }
}

// attention options (NULL: no sink, natural-log lse)
dsa_status check_opts(const dsa_attn_opts* o) {
  if (!o) return DSA_OK;
  if (o->sink && !al4(o->sink)) return DSA_ERR_ARG;
  if (o->lse_log2 != 0 && o->lse_log2 != 1) return DSA_ERR_ARG;
  return DSA_OK;
}

void apply_opts(MlaArgs& a, const dsa_attn_opts* o) {
  a.sink = o ? o->sink : nullptr;
  a.lse_log2 = o ? o->lse_log2 : 0;
}

KvDev make_kv(const dsa_kv_cache* kv) {
  KvDev d;
  d.data = static_cast<const uint8_t*>(kv->data);
  d.scales = kv->scales;
  d.pg = make_paging(kv->paging, kv->n_slots);
  return d;
}

struct MlaIn {
  const void* q;
  int64_t ld_q;
  const dsa_kv_cache* kv;
  const int32_t* idx;
  int64_t ld_idx;
  int32_t n_idx;
  const dsa_kv_cache* extra_kv;
  const int32_t* extra_idx;
  int64_t ld_extra;
  int32_t n_extra;
  int32_t T;
  const int32_t* row_req;
  int32_t n_req;
  int32_t H, d_qk, d_v;
  float softmax_scale;
  void* out;
  int64_t ld_out;
  float* lse;
  const dsa_attn_opts* opts;
};

dsa_status check_mla(const MlaIn& m) {
  if (m.T < 0 || m.H <= 0 || m.n_idx < 0 || m.n_extra < 0) return DSA_ERR_ARG;
  if (m.T > 65535) return DSA_ERR_UNSUPPORTED;
  if (m.d_v != 512) return DSA_ERR_UNSUPPORTED;
  if (m.d_qk != 512 && m.d_qk != 576) return DSA_ERR_UNSUPPORTED;
  if (!std::isfinite(m.softmax_scale)) return DSA_ERR_ARG;
  if (m.T == 0) return DSA_OK;
  if (!m.q || !al16(m.q) || m.ld_q < (int64_t)m.H * m.d_qk || m.ld_q % 8) return DSA_ERR_ARG;
  if (!m.out || !al16(m.out) || m.ld_out < (int64_t)m.H * m.d_v || m.ld_out % 8) return DSA_ERR_ARG;
  if (m.lse && !al4(m.lse)) return DSA_ERR_ARG;
  dsa_status s = check_opts(m.opts);
  if (s != DSA_OK) return s;
  s = check_kv(m.kv, m.d_qk);
  if (s != DSA_OK) return s;
  if (m.n_idx > 0 && (!m.idx || !al4(m.idx) || m.ld_idx < m.n_idx)) return DSA_ERR_ARG;
  if (m.n_extra > 0) {
    if (!m.extra_idx || !al4(m.extra_idx) || m.ld_extra < m.n_extra) return DSA_ERR_ARG;
    s = check_kv(m.extra_kv, m.d_qk);
    if (s != DSA_OK) return s;
    if (m.extra_kv->format != m.kv->format) return DSA_ERR_UNSUPPORTED;
  }
  return DSA_OK;
}

dsa_status run_mla(const MlaIn& m, bool decode, void* ws, size_t ws_bytes, hipStream_t st) {
  if (m.T == 0) return DSA_OK;
  const int ntot = m.n_idx + m.n_extra;
  const MlaPlan p = plan_mla(m.T, m.H, ntot, decode);
  if (!plan_ok(m.H, p)) return DSA_ERR_UNSUPPORTED;
  MlaArgs a;
  memset(&a, 0, sizeof(a));
  a.q = static_cast<const uint16_t*>(m.q);
  a.ld_q = m.ld_q;
  a.kv[0] = make_kv(m.kv);
  a.kv[1] = m.n_extra > 0 ? make_kv(m.extra_kv) : a.kv[0];
  a.idx[0] = m.idx;
  a.idx[1] = m.n_extra > 0 ? m.extra_idx : m.idx;
  a.ld_idx[0] = m.ld_idx;
  a.ld_idx[1] = m.n_extra > 0 ? m.ld_extra : m.ld_idx;
  a.n_idx[0] = m.n_idx;
  a.n_idx[1] = m.n_extra;
  a.row_req = m.row_req;
  a.n_req = m.n_req;
  a.H = m.H;
  a.Hp = heads_padded(m.H);
  a.n_split = p.n_split;
  a.rows_per_split = p.rows_per_split;
  a.scale_log2 = m.softmax_scale * kLog2e;
  a.out = static_cast<uint16_t*>(m.out);
  a.ld_out = m.ld_out;
  a.lse = m.lse;
  apply_opts(a, m.opts);
  if (p.n_split > 1) {
    const int64_t need = kHeaderBytes + mla_ws_bytes(m.T, m.H, ntot, decode);
    if (!ws || (int64_t)ws_bytes < need || !al16(ws)) return DSA_ERR_WORKSPACE;
    uint8_t* w = static_cast<uint8_t*>(ws);
    Carve cv;
    a.part_o = reinterpret_cast<float*>(w + cv.take((int64_t)m.T * a.Hp * p.n_split * 512 * 4));
    a.part_ml = reinterpret_cast<float*>(w + cv.take((int64_t)m.T * a.Hp * p.n_split * 8));
  }
  const int fmt = kv_fmt(m.kv);
  set_mla_row(m.T, m.H, m.n_idx, m.n_extra, fmt, m.d_qk, decode, p);
  dsa_status s = hip_status(timed("sparse_mla", st, [&] { return launch_sparse_mla(a, fmt, m.d_qk, p.ht, p.nbuf, m.T, st); }));
  if (s == DSA_OK && p.n_split > 1)
    s = hip_status(timed("mla_combine", st, [&] { return launch_mla_combine(a, m.T, st); }));
  return s;
}

// ---------------------------------------------------------------- top-k driver
struct TopkIn {
  const float* logits;
  int64_t ld_logits;
  const dsa_rows* rows;
  int32_t topk;
  int32_t* indices;
  int64_t ld_idx;
  int32_t* lens;
};

dsa_status check_topk(const TopkIn& k) {
  dsa_status s = check_rows(k.rows);
  if (s != DSA_OK) return s;
  if (k.topk < 1) return DSA_ERR_ARG;
  if (k.topk > 65536) return DSA_ERR_UNSUPPORTED;
  if (k.rows->n_max > kMaxChunks * kTopkChunk) return DSA_ERR_UNSUPPORTED;
  if (k.rows->T == 0) return DSA_OK;
  if (!k.logits || !al4(k.logits) || k.ld_logits < k.rows->n_max) return DSA_ERR_ARG;
  if (!k.indices || !al4(k.indices) || k.ld_idx < k.topk || !k.lens || !al4(k.lens)) return DSA_ERR_ARG;
  return DSA_OK;
}

// Long rows, in batches of kMaxLongRows rows: [first-digit histogram] -> filter -> finalize.
dsa_status run_topk_long(const TopkArgs& a, const dsa_rows& r, bool hist_ready, hipStream_t st) {
  set_row("T=%d n_max=%d topk=%d: long rows, batches of %d rows, %d chunks of %d, first digit %s", r.T,
          r.n_max, a.topk, kMaxLongRows, (r.n_max + kTopkChunk - 1) / kTopkChunk, kTopkChunk,
          hist_ready ? "from the score kernel" : "by its own kernel");
  for (int r0 = 0; r0 < r.T; r0 += kMaxLongRows) {
    const int nb = std::min(kMaxLongRows, r.T - r0);
    TopkArgs b = a;
    b.logits = a.logits + (int64_t)r0 * a.ld_logits;
    b.row_len = r.row_len + r0;
    b.indices = a.indices + (int64_t)r0 * a.ld_idx;
    b.lens = a.lens + r0;
    dsa_status s = DSA_OK;
    if (!hist_ready) s = hip_status(timed("topk_hist", st, [&] { return launch_topk_hist(b, nb, st); }));
    if (s == DSA_OK) s = hip_status(timed("topk_filter", st, [&] { return launch_topk_filter(b, nb, st); }));
    if (s == DSA_OK) s = hip_status(timed("topk_finalize", st, [&] { return launch_topk_finalize(b, nb, st); }));
    if (s != DSA_OK) return s;
  }
  return DSA_OK;
}

// hist_ready: the first-digit histogram of rows [0, T) was already accumulated (fused in the
// score kernel; only when T <= kMaxLongRows).
dsa_status run_topk(const TopkIn& k, bool hist_ready, void* ws, size_t ws_bytes, hipStream_t st) {
  const dsa_rows& r = *k.rows;
  if (r.T == 0) return DSA_OK;
  TopkArgs a;
  memset(&a, 0, sizeof(a));
  a.logits = k.logits;
  a.ld_logits = k.ld_logits;
  a.row_len = r.row_len;
  a.n_max = r.n_max;
  a.topk = k.topk;
  a.indices = k.indices;
  a.ld_idx = k.ld_idx;
  a.lens = k.lens;
  if (r.n_max <= kTopkLdsMax) {
    set_row("T=%d n_max=%d topk=%d: one workgroup per row, keys in registers (capacity %d)", r.T, r.n_max, k.topk,
            r.n_max <= 8704 ? 8704 : kTopkLdsMax);
    return hip_status(timed("topk_lds", st, [&] { return launch_topk_lds(a, r.T, st); }));
  }
  const int64_t need = kHeaderBytes + topk_ws_bytes(r.T, r.n_max);
  if (!ws || (int64_t)ws_bytes < need || !al16(ws)) return DSA_ERR_WORKSPACE;
  Carve cv;
  carve_topk(a, cv, static_cast<uint8_t*>(ws), r.T, r.n_max);
  return run_topk_long(a, r, hist_ready, st);
}

// ---------------------------------------------------------------- scores driver
struct ScoreIn {
  const void* q_idx;
  int64_t ld_q_idx;
  const float* w;
  int64_t ld_w;
  const dsa_key_cache* keys;
  const dsa_rows* rows;
  int32_t Hi, di;
  float index_scale;
  float* logits;
  int64_t ld_logits;
};

dsa_status check_scores(const ScoreIn& s) {
  dsa_status st = check_rows(s.rows);
  if (st != DSA_OK) return st;
  if (s.Hi < 1 || s.di < 1) return DSA_ERR_ARG;
  if (s.Hi > 64 || (s.di != 64 && s.di != 128)) return DSA_ERR_UNSUPPORTED;
  if (!std::isfinite(s.index_scale)) return DSA_ERR_ARG;
  if (!s.keys) return DSA_ERR_ARG;
  if (s.keys->dtype != DSA_KEY_BF16 && s.keys->dtype != DSA_KEY_FP8) return DSA_ERR_UNSUPPORTED;
  if (!s.keys->data || !al16(s.keys->data)) return DSA_ERR_ARG;
  if (s.keys->dtype == DSA_KEY_FP8 && (!s.keys->scale || !al4(s.keys->scale))) return DSA_ERR_ARG;
  st = check_paging(s.keys->paging, s.keys->n_slots);
  if (st != DSA_OK) return st;
  if (s.rows->T == 0) return DSA_OK;
  if (!s.q_idx || !al16(s.q_idx) || s.ld_q_idx < (int64_t)s.Hi * s.di || s.ld_q_idx % 8) return DSA_ERR_ARG;
  if (!s.w || !al4(s.w) || s.ld_w < s.Hi) return DSA_ERR_ARG;
  if (!s.logits || !al4(s.logits) || s.ld_logits < s.rows->n_max) return DSA_ERR_ARG;
  return DSA_OK;
}

// Many rows that share requests (more rows than requests: a prefill, an extend chunk,
// speculative verification): scored by the kernel whose workgroups share each key tile among
// 4 rows. Otherwise one row per workgroup.
bool shared_key_rows(const dsa_rows& r, const dsa_key_cache& k) {
  return r.row_req != nullptr && r.T >= kPrefillMinRows && r.T > r.n_req && k.dtype == DSA_KEY_BF16 &&
         k.n_slots <= INT32_MAX;
}

dsa_status run_scores(const ScoreIn& s, uint32_t* hist, hipStream_t st) {
  const dsa_rows& r = *s.rows;
  if (r.T == 0 || r.n_max == 0) return DSA_OK;
  ScoreArgs a;
  memset(&a, 0, sizeof(a));
  a.q_idx = static_cast<const uint16_t*>(s.q_idx);
  a.ld_q = s.ld_q_idx;
  a.w = s.w;
  a.ld_w = s.ld_w;
  a.keys = s.keys->data;
  a.key_scale = s.keys->scale;
  a.pg = make_paging(s.keys->paging, s.keys->n_slots);
  a.row_req = r.row_req;
  a.row_len = r.row_len;
  a.n_max = r.n_max;
  a.Hi = s.Hi;
  a.index_scale = s.index_scale;
  a.n_req = r.n_req;
  a.logits = s.logits;
  a.ld_logits = s.ld_logits;
  a.hist = hist;
  const bool shared = hist == nullptr && shared_key_rows(r, *s.keys);
  set_row("T=%d n_max=%d Hi=%d di=%d keys %s, page %d%s: %s", r.T, r.n_max, s.Hi, s.di,
          s.keys->dtype == DSA_KEY_FP8 ? "fp8" : "bf16", (int)s.keys->paging.page_size,
          s.keys->paging.block_table ? " (table)" : " (packed)",
          shared ? "rows sharing keys, 4 rows per workgroup" :
          hist ? "one row per workgroup, first top-k digit counted" : "one row per workgroup");
  if (shared)
    return hip_status(timed("index_scores_prefill", st, [&] { return launch_index_scores_prefill(a, s.di, r.T, st); }));
  return hip_status(timed(hist ? "index_scores_hist" : "index_scores", st, [&] {
    return launch_index_scores(a, s.di, s.keys->dtype == DSA_KEY_FP8, hist != nullptr, r.T, st);
  }));
}


// ---------------------------------------------------------------- the fused layer
struct DecodeIn {
  const void* q;
  int64_t ld_q;
  const void* q_idx;
  int64_t ld_q_idx;
  const float* w;
  int64_t ld_w;
  const dsa_key_cache* keys;
  const dsa_kv_cache* kv;
  const dsa_rows* rows;
  int32_t H, d_qk, d_v, Hi, di, topk;
  float index_scale, softmax_scale;
  void* out;
  int64_t ld_out;
  float* lse;
  const dsa_attn_opts* opts;
  int32_t* idx_out;
  int64_t ld_idx_out;
  int32_t* lens_out;
};

// Every argument check of the three steps, on the host (no HIP call); *need = workspace bytes.
dsa_status decode_check(const DecodeIn& d, size_t* need) {
  const dsa_rows* rows = d.rows;
  dsa_status s = check_rows(rows);
  if (s != DSA_OK) return s;
  if (d.topk < 1) return DSA_ERR_ARG;
  if (d.topk > 65536 || rows->n_max > kMaxChunks * kTopkChunk) return DSA_ERR_UNSUPPORTED;
  if (d.idx_out && (!al4(d.idx_out) || d.ld_idx_out < d.topk)) return DSA_ERR_ARG;
  if (d.lens_out && !al4(d.lens_out)) return DSA_ERR_ARG;
  const int T = rows->T;
  const int64_t ld = logits_ld(rows->n_max);
  // logits and indices are workspace-backed: stand-in pointers for the checks
  float* const dummy_f = reinterpret_cast<float*>(uintptr_t(256));
  const ScoreIn sc{d.q_idx, d.ld_q_idx, d.w, d.ld_w, d.keys, rows, d.Hi, d.di, d.index_scale, dummy_f, ld};
  s = check_scores(sc);
  if (s != DSA_OK) return s;
  const MlaIn m{d.q, d.ld_q, d.kv, reinterpret_cast<const int32_t*>(uintptr_t(256)), d.topk, d.topk,
                nullptr, nullptr, 0, 0, T, rows->row_req, rows->n_req, d.H, d.d_qk, d.d_v,
                d.softmax_scale, d.out, d.ld_out, d.lse, d.opts};
  s = check_mla(m);
  if (s != DSA_OK) return s;
  const dsa_problem pr{T, rows->n_max, d.topk, d.H, d.topk, 0};
  *need = dsa_workspace_size(DSA_ENTRY_DECODE, &pr);
  return *need == SIZE_MAX ? DSA_ERR_ARG : DSA_OK;
}

// The three steps on one stream over a checked problem (T > 0) and a workspace of at least
// the size decode_check gave, whose header is zero.
dsa_status decode_run(const DecodeIn& d, uint8_t* wsb, size_t ws_bytes, hipStream_t st) {
  const dsa_rows* rows = d.rows;
  const int T = rows->T;
  const int64_t ld = logits_ld(rows->n_max);
  Carve cv;
  float* logits = reinterpret_cast<float*>(wsb + cv.take((int64_t)T * ld * 4));
  int32_t* idx_ws = reinterpret_cast<int32_t*>(wsb + cv.take((int64_t)T * d.topk * 4));
  int32_t* lens_ws = reinterpret_cast<int32_t*>(wsb + cv.take((int64_t)T * 4));
  int32_t* idx = d.idx_out ? d.idx_out : idx_ws;
  const int64_t ld_idx = d.idx_out ? d.ld_idx_out : d.topk;
  int32_t* lens = d.lens_out ? d.lens_out : lens_ws;

  // step 1 (+ the first top-k digit when the long-row path will run and fits one batch)
  const bool long_rows = rows->n_max > kTopkLdsMax;
  // (rows that share their keys are scored by the shared-key kernel, which has no histogram)
  const bool fuse_hist = long_rows && T <= kMaxLongRows && !shared_key_rows(*rows, *d.keys);
  const ScoreIn sc{d.q_idx, d.ld_q_idx, d.w, d.ld_w, d.keys, rows, d.Hi, d.di, d.index_scale, logits, ld};
  dsa_status s = run_scores(sc, fuse_hist ? reinterpret_cast<uint32_t*>(wsb + kOffHist) : nullptr, st);
  if (s != DSA_OK) return s;
  // step 2: top-k; its candidate lists are carved after the regions above
  {
    if (!long_rows) {
      const TopkIn tk{logits, ld, rows, d.topk, idx, ld_idx, lens};
      s = run_topk(tk, false, nullptr, 0, st);
    } else {
      TopkArgs a;
      memset(&a, 0, sizeof(a));
      a.logits = logits;
      a.ld_logits = ld;
      a.row_len = rows->row_len;
      a.n_max = rows->n_max;
      a.topk = d.topk;
      a.indices = idx;
      a.ld_idx = ld_idx;
      a.lens = lens;
      carve_topk(a, cv, wsb, T, rows->n_max);
      s = run_topk_long(a, *rows, fuse_hist, st);
    }
    if (s != DSA_OK) return s;
  }
  // step 3: attention over the selection; split partials after our regions
  const bool decode = T <= 1024;
  const MlaPlan p = plan_mla(T, d.H, d.topk, decode);
  if (!plan_ok(d.H, p)) return DSA_ERR_UNSUPPORTED;
  MlaArgs a;
  memset(&a, 0, sizeof(a));
  a.q = static_cast<const uint16_t*>(d.q);
  a.ld_q = d.ld_q;
  a.kv[0] = make_kv(d.kv);
  a.kv[1] = a.kv[0];
  a.idx[0] = idx;
  a.idx[1] = idx;
  a.ld_idx[0] = ld_idx;
  a.ld_idx[1] = ld_idx;
  a.n_idx[0] = d.topk;
  a.n_idx[1] = 0;
  a.row_req = rows->row_req;
  a.n_req = rows->n_req;
  a.H = d.H;
  a.Hp = heads_padded(d.H);
  a.n_split = p.n_split;
  a.rows_per_split = p.rows_per_split;
  a.scale_log2 = d.softmax_scale * kLog2e;
  a.out = static_cast<uint16_t*>(d.out);
  a.ld_out = d.ld_out;
  a.lse = d.lse;
  apply_opts(a, d.opts);
  if (p.n_split > 1) {
    a.part_o = reinterpret_cast<float*>(wsb + cv.take((int64_t)T * a.Hp * p.n_split * 512 * 4));
    a.part_ml = reinterpret_cast<float*>(wsb + cv.take((int64_t)T * a.Hp * p.n_split * 8));
    if ((size_t)cv.off > ws_bytes) return DSA_ERR_WORKSPACE;
  }
  const int fmt = kv_fmt(d.kv);
  set_mla_row(T, d.H, d.topk, 0, fmt, d.d_qk, decode, p);
  s = hip_status(timed("sparse_mla", st, [&] { return launch_sparse_mla(a, fmt, d.d_qk, p.ht, p.nbuf, T, st); }));
  if (s == DSA_OK && p.n_split > 1)
    s = hip_status(timed("mla_combine", st, [&] { return launch_mla_combine(a, T, st); }));
  return s;
}

// ---------------------------------------------------------------- static scratch
// The workspace of dsa_decode_static: one file-scope device array, which every GPU the library
// runs on holds until the process ends. In host code `scratch` names a host-side stand-in; the
// device address of each GPU's copy comes from hipGetSymbolAddress, taken once per device with
// that device current, and only that address is ever handed to a kernel.
__device__ __align__(256) uint8_t scratch[DSA_STATIC_SCRATCH_BYTES];

struct StaticScratch {
  void* ptr = nullptr;     // this device's copy of `scratch`
  bool dirty = true;       // its header must be zeroed before the next use
};
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
StaticScratch g_scratch[kMaxDevices];

// The scratch of the device that `st` runs on (the current device for the null stream).
dsa_status static_scratch(hipStream_t st, StaticScratch** out) {
  int dev = -1;
  if (st ? hipStreamGetDevice(st, &dev) != hipSuccess : hipGetDevice(&dev) != hipSuccess) return DSA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return DSA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  StaticScratch& sc = g_scratch[dev];
  if (!sc.ptr) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return DSA_ERR_HIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return DSA_ERR_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev && hipSetDevice(cur) != hipSuccess) return DSA_ERR_HIP;
    if (e != hipSuccess || !p || ((uintptr_t)p & 255u)) return DSA_ERR_HIP;
    sc.ptr = p;
    sc.dirty = true;
  }
  *out = &sc;
  return DSA_OK;
}

}  // namespace

// ==================================================================== exported entry points
extern "C" {

int32_t dsa_abi_version(void) { return 7; }

dsa_status dsa_launch_override(int32_t head_tiles, int32_t n_split) {
  if (!(head_tiles == 0 || head_tiles == 1 || head_tiles == 2 || head_tiles == 4)) return DSA_ERR_ARG;
  if (n_split < 0 || n_split > 65535) return DSA_ERR_ARG;
  g_force_ht = head_tiles;
  g_force_split = n_split;
  return DSA_OK;
}
dsa_status dsa_kv_cache_write(const void* src, int64_t ld_src, int32_t n_tok, const int32_t* slots,
                              const dsa_kv_cache* kv, void* stream) {
  if (n_tok < 0 || !kv) return DSA_ERR_ARG;
  if (n_tok == 0) return DSA_OK;
  if (!src || !al16(src) || !slots || !al4(slots) || !kv->data || ld_src % 8) return DSA_ERR_ARG;
  if (kv->n_slots < 1) return DSA_ERR_ARG;
  CacheWriteArgs a;
  memset(&a, 0, sizeof(a));
  a.src = static_cast<const uint16_t*>(src);
  a.ld_src = ld_src;
  a.n_tok = n_tok;
  a.D = kv->d_nope + kv->d_rope;
  a.slots = slots;
  a.n_slots = kv->n_slots;
  a.data = static_cast<uint8_t*>(const_cast<void*>(kv->data));
  if (ld_src < a.D || kv->d_nope < 0 || kv->d_rope < 0) return DSA_ERR_ARG;
  int kind;
  switch (kv->format) {
    case DSA_KV_BF16:
      if (a.D % 8 || !al16(kv->data)) return DSA_ERR_ARG;
      kind = kCwBf16;
      break;
    case DSA_KV_FP8_UNIFORM:
      if (a.D % 64 || a.D > 4096) return DSA_ERR_UNSUPPORTED;
      if (!kv->scales || !al4(kv->scales) || !al16(kv->data)) return DSA_ERR_ARG;
      a.fscale = const_cast<float*>(kv->scales);
      a.group = 64;
      kind = kCwScaled;
      break;
    case DSA_KV_FP8_UNIFORM_FNUZ:
      if (a.D % 64 || a.D > 4096) return DSA_ERR_UNSUPPORTED;
      if (!kv->scales || !al4(kv->scales) || !al16(kv->data)) return DSA_ERR_ARG;
      a.fscale = const_cast<float*>(kv->scales);
      a.group = 64;
      kind = kCwScaledFnuz;
      break;
    case DSA_KV_FP8_DS_MLA:
      if (kv->d_nope != 448 || kv->d_rope != 64) return DSA_ERR_UNSUPPORTED;
      if (kv->paging.page_size < 1 || kv->n_slots % kv->paging.page_size || !al16(kv->data)) return DSA_ERR_ARG;
      a.page = kv->paging.page_size;
      kind = kCwDsMla;
      break;
    default:
      return DSA_ERR_ARG;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  set_row("%d token(s) of %d + %d columns into a %s cache", n_tok, kv->d_nope, kv->d_rope,
          kind == kCwBf16 ? "bf16" : kind == kCwDsMla ? "fp8_ds_mla" : kind == kCwScaledFnuz ? "fnuz fp8" : "fp8");
  return hip_status(timed("cache_write_kv", st, [&] { return launch_cache_write(a, kind, st); }));
}

dsa_status dsa_key_cache_write(const void* src, int64_t ld_src, int32_t n_tok, const int32_t* slots,
                               const dsa_key_cache* keys, int32_t di, void* stream) {
  if (n_tok < 0 || !keys) return DSA_ERR_ARG;
  if (di != 64 && di != 128) return DSA_ERR_UNSUPPORTED;
  if (n_tok == 0) return DSA_OK;
  if (!src || !al16(src) || !slots || !al4(slots) || !keys->data || !al16(keys->data)) return DSA_ERR_ARG;
  if (ld_src < di || ld_src % 8 || keys->n_slots < 1) return DSA_ERR_ARG;
  CacheWriteArgs a;
  memset(&a, 0, sizeof(a));
  a.src = static_cast<const uint16_t*>(src);
  a.ld_src = ld_src;
  a.n_tok = n_tok;
  a.D = di;
  a.slots = slots;
  a.n_slots = keys->n_slots;
  a.data = static_cast<uint8_t*>(const_cast<void*>(keys->data));
  int kind;
  if (keys->dtype == DSA_KEY_BF16) {
    kind = kCwBf16;
  } else if (keys->dtype == DSA_KEY_FP8) {
    if (!keys->scale || !al4(keys->scale)) return DSA_ERR_ARG;
    a.fscale = const_cast<float*>(keys->scale);
    a.group = di;
    kind = kCwScaled;
  } else {
    return DSA_ERR_ARG;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  set_row("%d key(s) of %d into a %s key cache", n_tok, di, kind == kCwBf16 ? "bf16" : "fp8");
  return hip_status(timed("cache_write_keys", st, [&] { return launch_cache_write(a, kind, st); }));
}


const char* dsa_status_string(int32_t status) {
  switch (status) {
    case DSA_OK: return "ok";
    case DSA_ERR_ARG: return "invalid argument (null pointer, bad shape, stride or alignment)";
    case DSA_ERR_UNSUPPORTED: return "unsupported shape or format (outside the compiled envelope)";
    case DSA_ERR_WORKSPACE: return "workspace missing or too small (see dsa_workspace_size)";
    case DSA_ERR_HIP: return "HIP launch failed";
    case DSA_ERR_SCRATCH_LIMIT:
      return "problem needs more than the static scratch of dsa_decode_static (DSA_STATIC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

size_t dsa_workspace_size(int32_t entry, const dsa_problem* p) {
  if (!p || p->T < 0 || p->n_max < 0 || p->topk < 0 || p->H < 0 || p->n_idx < 0) return SIZE_MAX;
  switch (entry) {
    case DSA_ENTRY_TOPK:
      return (size_t)(kHeaderBytes + topk_ws_bytes(p->T, p->n_max));
    case DSA_ENTRY_MLA_DECODE:
      return (size_t)(kHeaderBytes + mla_ws_bytes(p->T, p->H, p->n_idx, true));
    case DSA_ENTRY_MLA_PREFILL:
      return 0;
    case DSA_ENTRY_MLA_BACKWARD:
      if (p->H > 128) return SIZE_MAX;
      if (p->n_slots < 0) return SIZE_MAX;
      return (size_t)(kHeaderBytes + mla_bwd_ws_bytes(p->T, p->H, p->n_idx) +
                      (p->n_slots > 0 ? mla_bwd_owner_bytes(p->n_slots) : 0));
    case DSA_ENTRY_DECODE: {
      const int64_t ld = logits_ld(p->n_max);
      int64_t b = kHeaderBytes;
      b = align256(b + (int64_t)p->T * ld * 4);                 // logits
      b = align256(b + (int64_t)p->T * p->topk * 4);            // indices
      b = align256(b + (int64_t)p->T * 4);                      // lens
      b += topk_ws_bytes(p->T, p->n_max);
      b = align256(b);
      b += mla_ws_bytes(p->T, p->H, p->topk, p->T <= 1024);
      return (size_t)b;
    }
    default:
      return SIZE_MAX;
  }
}

dsa_status dsa_workspace_init(void* workspace, size_t ws_bytes, void* stream) {
  if (!workspace || !al16(workspace)) return DSA_ERR_ARG;
  if ((int64_t)ws_bytes < kHeaderBytes) return DSA_ERR_WORKSPACE;
  return hip_status(launch_fill_zero(workspace, ws_bytes, static_cast<hipStream_t>(stream)));
}

dsa_status dsa_index_scores(const void* q_idx, int64_t ld_q_idx, const float* w, int64_t ld_w,
                            const dsa_key_cache* keys, const dsa_rows* rows, int32_t Hi,
                            int32_t di, float index_scale, float* logits, int64_t ld_logits,
                            void* stream) {
  ScoreIn s{q_idx, ld_q_idx, w, ld_w, keys, rows, Hi, di, index_scale, logits, ld_logits};
  dsa_status st = check_scores(s);
  if (st != DSA_OK) return st;
  return run_scores(s, nullptr, static_cast<hipStream_t>(stream));
}

dsa_status dsa_topk(const float* logits, int64_t ld_logits, const dsa_rows* rows, int32_t topk,
                    int32_t* indices, int64_t ld_idx, int32_t* lens, void* workspace,
                    size_t ws_bytes, void* stream) {
  TopkIn k{logits, ld_logits, rows, topk, indices, ld_idx, lens};
  dsa_status st = check_topk(k);
  if (st != DSA_OK) return st;
  return run_topk(k, false, workspace, ws_bytes, static_cast<hipStream_t>(stream));
}

dsa_status dsa_sparse_mla_decode(const void* q, int64_t ld_q, const dsa_kv_cache* kv,
                                 const int32_t* idx, int64_t ld_idx, int32_t n_idx,
                                 const dsa_kv_cache* extra_kv, const int32_t* extra_idx,
                                 int64_t ld_extra, int32_t n_extra, int32_t B, int32_t H,
                                 int32_t d_qk, int32_t d_v, float softmax_scale, void* out,
                                 int64_t ld_out, float* lse, const dsa_attn_opts* opts,
                                 void* workspace, size_t ws_bytes, void* stream) {
  MlaIn m{q, ld_q, kv, idx, ld_idx, n_idx, extra_kv, extra_idx, ld_extra, n_extra, B, nullptr,
          B, H, d_qk, d_v, softmax_scale, out, ld_out, lse, opts};
  dsa_status st = check_mla(m);
  if (st != DSA_OK) return st;
  return run_mla(m, true, workspace, ws_bytes, static_cast<hipStream_t>(stream));
}

dsa_status dsa_sparse_mla_prefill(const void* q, int64_t ld_q, const dsa_kv_cache* kv,
                                  const int32_t* idx, int64_t ld_idx, int32_t n_idx,
                                  const dsa_kv_cache* extra_kv, const int32_t* extra_idx,
                                  int64_t ld_extra, int32_t n_extra, const dsa_rows* rows,
                                  int32_t H, int32_t d_qk, int32_t d_v, float softmax_scale,
                                  void* out, int64_t ld_out, float* lse,
                                  const dsa_attn_opts* opts, void* workspace, size_t ws_bytes,
                                  void* stream) {
  dsa_status st = check_rows(rows);
  if (st != DSA_OK) return st;
  MlaIn m{q, ld_q, kv, idx, ld_idx, n_idx, extra_kv, extra_idx, ld_extra, n_extra, rows->T,
          rows->row_req, rows->n_req, H, d_qk, d_v, softmax_scale, out, ld_out, lse, opts};
  st = check_mla(m);
  if (st != DSA_OK) return st;
  return run_mla(m, false, workspace, ws_bytes, static_cast<hipStream_t>(stream));
}

dsa_status dsa_sparse_mla_backward(const void* q, int64_t ld_q, const dsa_kv_cache* kv,
                                   const int32_t* idx, int64_t ld_idx, int32_t n_idx,
                                   const dsa_rows* rows, int32_t H, int32_t d_qk, int32_t d_v,
                                   float softmax_scale, const void* out, int64_t ld_out,
                                   const float* lse, const void* dout, int64_t ld_dout,
                                   const dsa_attn_opts* opts, float* dq, int64_t ld_dq,
                                   float* dkv, float* dsink, void* workspace, size_t ws_bytes,
                                   void* stream) {
  dsa_status st = check_rows(rows);
  if (st != DSA_OK) return st;
  if (H <= 0 || n_idx < 0) return DSA_ERR_ARG;
  if (H > 128 || d_v != 512 || (d_qk != 512 && d_qk != 576)) return DSA_ERR_UNSUPPORTED;
  if (!std::isfinite(softmax_scale)) return DSA_ERR_ARG;
  st = check_opts(opts);
  if (st != DSA_OK) return st;
  st = check_kv(kv, d_qk);
  if (st != DSA_OK) return st;
  if (kv->format != DSA_KV_BF16) return DSA_ERR_UNSUPPORTED;
  if (dsink && (!opts || !opts->sink || !al4(dsink))) return DSA_ERR_ARG;
  const int T = rows->T;
  if (T == 0) return DSA_OK;
  if (!q || !al16(q) || ld_q < (int64_t)H * d_qk || ld_q % 8) return DSA_ERR_ARG;
  if (!out || !al16(out) || ld_out < (int64_t)H * d_v || ld_out % 8) return DSA_ERR_ARG;
  if (!dout || !al16(dout) || ld_dout < (int64_t)H * d_v || ld_dout % 8) return DSA_ERR_ARG;
  if (!lse || !al4(lse)) return DSA_ERR_ARG;
  if (n_idx > 0 && (!idx || !al4(idx) || ld_idx < n_idx)) return DSA_ERR_ARG;
  if (!dq || !al16(dq) || ld_dq < (int64_t)H * d_qk || ld_dq % 4) return DSA_ERR_ARG;
  if (!dkv || !al4(dkv)) return DSA_ERR_ARG;
  const int64_t need = kHeaderBytes + mla_bwd_ws_bytes(T, H, n_idx);
  if (!workspace || (int64_t)ws_bytes < need || !al16(workspace)) return DSA_ERR_WORKSPACE;
  MlaBwdArgs a;
  memset(&a, 0, sizeof(a));
  a.q = static_cast<const uint16_t*>(q);
  a.ld_q = ld_q;
  a.kv = make_kv(kv);
  a.idx = idx;
  a.ld_idx = ld_idx;
  a.n_idx = n_idx;
  a.row_req = rows->row_req;
  a.n_req = rows->n_req;
  a.H = H;
  a.Hp = heads_padded_bwd(H);
  a.scale = softmax_scale;
  a.scale_log2 = softmax_scale * kLog2e;
  a.out = static_cast<const uint16_t*>(out);
  a.ld_out = ld_out;
  a.lse = lse;
  a.lse_log2 = opts ? opts->lse_log2 : 0;
  a.dout = static_cast<const uint16_t*>(dout);
  a.ld_dout = ld_dout;
  a.sink = opts ? opts->sink : nullptr;
  a.dq = dq;
  a.ld_dq = ld_dq;
  a.dkv = dkv;
  a.dsink = dsink;
  {
    uint8_t* w = static_cast<uint8_t*>(workspace);
    Carve cv;
    const int64_t e = (int64_t)T * n_idx;
    a.ws_dz = reinterpret_cast<uint16_t*>(w + cv.take(e * a.Hp * 2));
    a.ws_p = reinterpret_cast<uint16_t*>(w + cv.take(e * a.Hp * 2));
    a.ws_slot = reinterpret_cast<int32_t*>(w + cv.take(e * 4));
    a.nsplit = bwd_splits(T, a.Hp, n_idx);
    if (a.nsplit > 1) a.ws_dqp = reinterpret_cast<float*>(w + cv.take((int64_t)(a.nsplit - 1) * T * a.Hp * 576 * 4));
    // the owner map when the workspace has room for one over this cache's slots
    const int64_t ob = mla_bwd_owner_bytes(kv->n_slots);
    if ((a.Hp == 32 || a.Hp == 64) && n_idx > 0 && kv->n_slots <= INT32_MAX && (int64_t)ws_bytes >= need + ob) {
      a.ws_owner = reinterpret_cast<int32_t*>(w + cv.take(ob));
      a.n_slots = kv->n_slots;
    }
  }
  hipStream_t hs = static_cast<hipStream_t>(stream);
  set_row("T=%d H=%d (padded %d) list %d d_qk=%d: one workgroup per (row, %d heads, list part of %d), dKV over "
          "all heads%s", T, H, (int)a.Hp, n_idx, d_qk, a.Hp == 16 ? 16 : 32, (int)a.nsplit,
          a.ws_owner ? ", owner map (plain adds for singly named slots)" : "");
  dsa_status s = hip_status(timed("sparse_mla_bwd", hs, [&] { return launch_sparse_mla_bwd(a, d_qk, T, hs); }));
  if (s == DSA_OK && (a.ws_owner || a.nsplit > 1))
    s = hip_status(timed("sparse_mla_bwd_mid", hs, [&] { return launch_sparse_mla_bwd_mid(a, d_qk, T, hs); }));
  if (s == DSA_OK)
    s = hip_status(timed("sparse_mla_bwd_dkv", hs, [&] { return launch_sparse_mla_bwd_dkv(a, d_qk, T, hs); }));
  return s;
}

dsa_status dsa_decode(const void* q, int64_t ld_q, const void* q_idx, int64_t ld_q_idx,
                      const float* w, int64_t ld_w, const dsa_key_cache* keys,
                      const dsa_kv_cache* kv, const dsa_rows* rows, int32_t H, int32_t d_qk,
                      int32_t d_v, int32_t Hi, int32_t di, int32_t topk, float index_scale,
                      float softmax_scale, void* out, int64_t ld_out, float* lse,
                      const dsa_attn_opts* opts, int32_t* idx_out, int64_t ld_idx_out,
                      int32_t* lens_out,
                      void* workspace, size_t ws_bytes, void* stream) {
  const DecodeIn d{q, ld_q, q_idx, ld_q_idx, w, ld_w, keys, kv, rows, H, d_qk, d_v, Hi, di, topk,
                   index_scale, softmax_scale, out, ld_out, lse, opts, idx_out, ld_idx_out, lens_out};
  size_t need = 0;
  dsa_status s = decode_check(d, &need);
  if (s != DSA_OK || rows->T == 0) return s;
  if (!workspace || !al16(workspace) || ws_bytes < need) return DSA_ERR_WORKSPACE;
  return decode_run(d, static_cast<uint8_t*>(workspace), ws_bytes, static_cast<hipStream_t>(stream));
}

dsa_status dsa_decode_static(const void* q, int64_t ld_q, const void* q_idx, int64_t ld_q_idx,
                             const float* w, int64_t ld_w, const dsa_key_cache* keys,
                             const dsa_kv_cache* kv, const dsa_rows* rows, int32_t H,
                             int32_t d_qk, int32_t d_v, int32_t Hi, int32_t di, int32_t topk,
                             float index_scale, float softmax_scale, void* out, int64_t ld_out,
                             float* lse, const dsa_attn_opts* opts, int32_t* idx_out,
                             int64_t ld_idx_out, int32_t* lens_out, void* stream) {
  const DecodeIn d{q, ld_q, q_idx, ld_q_idx, w, ld_w, keys, kv, rows, H, d_qk, d_v, Hi, di, topk,
                   index_scale, softmax_scale, out, ld_out, lse, opts, idx_out, ld_idx_out, lens_out};
  size_t need = 0;
  dsa_status s = decode_check(d, &need);
  if (s != DSA_OK || rows->T == 0) return s;
  if (need > (size_t)DSA_STATIC_SCRATCH_BYTES) return DSA_ERR_SCRATCH_LIMIT;
  hipStream_t st = static_cast<hipStream_t>(stream);
  StaticScratch* sc = nullptr;
  s = static_scratch(st, &sc);
  if (s != DSA_OK) return s;
  if (sc->dirty) {                                   // first call on this device, or after a failure
    s = hip_status(launch_fill_zero(sc->ptr, (size_t)kHeaderBytes, st));
    if (s != DSA_OK) return s;
    sc->dirty = false;
  }
  s = decode_run(d, static_cast<uint8_t*>(sc->ptr), (size_t)DSA_STATIC_SCRATCH_BYTES, st);
  if (s == DSA_ERR_HIP) sc->dirty = true;            // the control words may not be back at zero
  return s;
}

dsa_status dsa_profile_enable(int32_t on) {
  g_prof = on != 0;
  return DSA_OK;
}

int32_t dsa_profile_collect(dsa_kernel_time* out, int32_t max_entries) {
  if (!out || max_entries < 0) return DSA_ERR_ARG;
  int32_t n = 0;
  dsa_status st = DSA_OK;
  for (const ProfRec& r : g_recs) {
    float ms = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) {
      st = DSA_ERR_HIP;
    } else {
      int32_t i = 0;
      while (i < n && strncmp(out[i].name, r.name, sizeof(out[i].name)) != 0) ++i;
      if (i == n && n < max_entries) {
        memset(&out[n], 0, sizeof(out[n]));
        strncpy(out[n].name, r.name, sizeof(out[n].name) - 1);
        out[n].min_ms = ms;
        out[n].max_ms = ms;
        ++n;
      }
      if (i < n) {
        out[i].count += 1;
        out[i].total_ms += ms;
        out[i].min_ms = std::min(out[i].min_ms, ms);
        out[i].max_ms = std::max(out[i].max_ms, ms);
      }
    }
    g_event_pool.push_back(r.a);
    g_event_pool.push_back(r.b);
  }
  g_recs.clear();
  return st == DSA_OK ? n : (int32_t)st;
}

}  // extern "C"
