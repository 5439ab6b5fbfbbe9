// Sparse absorbed-MLA attention over gathered latent rows, gfx950 MFMA.
//
// For query row t and head h, over the listed cache rows c_i (entries -1 contribute nothing):
//   out[t,h] = sum_i softmax_i(softmax_scale * q[t,h] . c_i) * c_i[0:512],  lse = ln sum_i e^(.)
// Rows are 512 latent + 64 RoPE bf16 (tokenspeed PR 664 "gfx950 Gluon bf16 MLA decode and
// prefill kernels"), or fp8 rows of aiter PR 4382 "Paged Sparse Attention Gluon Kernel"
// (uniform pool: fp8 * fp32 scale per 64 columns; fp8_ds_mla: 448 NoPE fp8 * 2^(e-127) per 64
// columns + 64 RoPE bf16, page-planar 584 bytes/token). -1 entries are masked from the
// original list while their rows are never read (radixark/miles PR 3608, "What", padding).
// A second list (extra) into a second cache shares the softmax (PR 4382, two-loop layout).
//
// Workgroup = 4 waves. A wave owns 16 heads; HT head tiles share each gathered block, and the
// remaining 4/HT waves form independent row streams that are merged through LDS at the end.
// Per 32-row block a stream gathers its rows into LDS as bf16 (fp8 dequantised on the way),
// then each wave computes
//   S^T[32 rows x 16 heads] = K Q^T   (A = rows from LDS, B = q held in registers),
// an online softmax in base 2, and
//   O^T[512 x 16 heads] += V^T P^T   (A = V^T read from LDS and transposed 8x8 in registers,
//                                      B = P^T straight from S^T's accumulator layout).
// With the 16x16x32 layout, S^T's accumulator rows (4 per lane group, two 16-row tiles) are
// exactly the k-slots of P^T as a B operand, so P never crosses lanes.
// Splits (decode): each workgroup covers rows_per_split entries of the row's list, writes an
// un-normalised partial (o, m, l), and the last workgroup of the (row, head group) merges
// them (split-KV + LSE merge of PR 664).
#include "common.hpp"
#include "kernels.hpp"

namespace dsa {

constexpr int kNB = 32;     // rows per block
constexpr int kDV = 512;    // value width

template <int FMT, int DQK>
struct RowGeom {
  static constexpr int kElems = DQK + 8;                       // padded bf16 row in LDS
  // 16-byte work units per row and what one unit produces
  static constexpr int kUnits = FMT == kFmtBf16 ? DQK / 8 : (FMT == kFmtUniform ? DQK / 16 : 36);
};

// One unit of a gathered row: global -> (dequant) -> LDS bf16.
template <int FMT, int DQK>
__device__ __forceinline__ void stage_unit(const KvDev& kv, int64_t slot, bool valid, int u,
                                           uint16_t* lrow) {
  if constexpr (FMT == kFmtBf16) {
    u32x4_t v = u32x4_t{0u, 0u, 0u, 0u};
    if (valid) v = *reinterpret_cast<const u32x4_t*>(kv.data + (slot * DQK + 8 * u) * 2);
    *reinterpret_cast<u32x4_t*>(lrow + 8 * u) = v;
  } else if constexpr (FMT == kFmtUniform) {
    u32x4_t lo = u32x4_t{0u, 0u, 0u, 0u}, hi = lo;
    if (valid) {
      const u32x4_t raw = *reinterpret_cast<const u32x4_t*>(kv.data + slot * DQK + 16 * u);
      const float sc = kv.scales[slot * (DQK / 64) + (16 * u) / 64];
      float f[16];
      fp8x4_to_f32(raw[0], f);
      fp8x4_to_f32(raw[1], f + 4);
      fp8x4_to_f32(raw[2], f + 8);
      fp8x4_to_f32(raw[3], f + 12);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        lo[i] = pack_bf16_rne(f[2 * i] * sc, f[2 * i + 1] * sc);
        hi[i] = pack_bf16_rne(f[8 + 2 * i] * sc, f[8 + 2 * i + 1] * sc);
      }
    }
    *reinterpret_cast<u32x4_t*>(lrow + 16 * u) = lo;
    *reinterpret_cast<u32x4_t*>(lrow + 16 * u + 8) = hi;
  } else {  // fp8_ds_mla
    const int P = kv.pg.page;
    int64_t page, pos;
    if (kv.pg.page_shift >= 0) { page = slot >> kv.pg.page_shift; pos = slot & (P - 1); }
    else { page = slot / P; pos = slot - page * P; }
    const uint8_t* pbase = kv.data + page * (int64_t)P * 584;
    const uint8_t* tok = pbase + pos * 576;
    if (u < 28) {
      u32x4_t lo = u32x4_t{0u, 0u, 0u, 0u}, hi = lo;
      if (valid) {
        const u32x4_t raw = *reinterpret_cast<const u32x4_t*>(tok + 16 * u);
        const float sc = ue8m0_scale(pbase[(int64_t)P * 576 + pos * 8 + (u >> 2)]);
        float f[16];
        fp8x4_to_f32(raw[0], f);
        fp8x4_to_f32(raw[1], f + 4);
        fp8x4_to_f32(raw[2], f + 8);
        fp8x4_to_f32(raw[3], f + 12);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          lo[i] = pack_bf16_exact(f[2 * i] * sc, f[2 * i + 1] * sc);
          hi[i] = pack_bf16_exact(f[8 + 2 * i] * sc, f[8 + 2 * i + 1] * sc);
        }
      }
      *reinterpret_cast<u32x4_t*>(lrow + 16 * u) = lo;
      *reinterpret_cast<u32x4_t*>(lrow + 16 * u + 8) = hi;
    } else {
      u32x4_t v = u32x4_t{0u, 0u, 0u, 0u};
      if (valid) v = *reinterpret_cast<const u32x4_t*>(tok + 448 + 16 * (u - 28));
      *reinterpret_cast<u32x4_t*>(lrow + 448 + 8 * (u - 28)) = v;
    }
  }
}

template <int FMT, int DQK, int HT, bool SPLIT>
__global__ __launch_bounds__(256) void k_sparse_mla(MlaArgs a) {
  constexpr int RS = 4 / HT;
  constexpr int KS = DQK / 32;
  constexpr int RE = RowGeom<FMT, DQK>::kElems;
  constexpr int UN = RowGeom<FMT, DQK>::kUnits;
  constexpr int NLANE = 64 * HT;                 // lanes that gather one stream's block
  __shared__ __align__(16) uint16_t s_rows[RS][kNB][RE];
  __shared__ int64_t s_slot[RS][kNB];
  __shared__ int32_t s_info[RS][kNB];            // bit0: valid, bit1: extra list
  __shared__ uint32_t s_flag;

  const int t = blockIdx.z;
  const int hg = blockIdx.y;
  const int split = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int ht = wave % HT;
  const int rs = wave / HT;
  const int g = lane >> 4;
  const int c = lane & 15;
  const int b = min(max(a.row_req ? a.row_req[t] : t, 0), a.n_req - 1);
  const int head0 = (hg * HT + ht) * 16;
  const int n0 = a.n_idx[0];
  const int ntot = n0 + a.n_idx[1];
  const int u_begin = split * a.rows_per_split;
  const int u_end = min(ntot, u_begin + a.rows_per_split);
  const int nblk = u_end > u_begin ? (u_end - u_begin + kNB - 1) / kNB : 0;
  const int iters = (nblk + RS - 1) / RS;

  u32x4_t qb[KS];
  {
    const uint16_t* qp = a.q + (int64_t)t * a.ld_q + (int64_t)(head0 + c) * DQK + 8 * g;
#pragma unroll
    for (int kb = 0; kb < KS; ++kb) qb[kb] = *reinterpret_cast<const u32x4_t*>(qp + 32 * kb);
  }

  float m_run = -INFINITY;
  float l_run = 0.f;
  f32x4_t o[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[i][e] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int it = 0; it < iters; ++it) {
    const int blk = it * RS + rs;
    const bool active = blk < nblk;
    const int sl = ht * 64 + lane;
    // ---- phase A: resolve the block's list entries to cache slots
    if (active && sl < kNB) {
      const int uu = u_begin + blk * kNB + sl;
      int info = 0;
      int64_t slot = 0;
      if (uu < u_end) {
        const int li = uu < n0 ? 0 : 1;
        const int j = uu - (li ? n0 : 0);
        const int e = a.idx[li][(int64_t)t * a.ld_idx[li] + j];
        if (e >= 0) {
          slot = slot_of(a.kv[li].pg, b, e);
          info = 1 | (li << 1);
        }
      }
      s_slot[rs][sl] = slot;
      s_info[rs][sl] = info;
    }
    __syncthreads();
    // ---- phase B: gather + dequantise into LDS
    if (active) {
      constexpr int TOT = kNB * UN;
      constexpr int BATCH = 4;
      for (int u0 = sl; u0 < TOT; u0 += NLANE * BATCH) {
#pragma unroll
        for (int q = 0; q < BATCH; ++q) {
          const int uid = u0 + q * NLANE;
          if (uid < TOT) {
            const int r = uid / UN;
            const int u = uid - r * UN;
            const int info = s_info[rs][r];
            stage_unit<FMT, DQK>(a.kv[(info >> 1) & 1], s_slot[rs][r], info & 1, u, &s_rows[rs][r][0]);
          }
        }
      }
    }
    __syncthreads();
    // ---- phase C: S^T = K Q^T, online softmax, O^T += V^T P^T
    if (active) {
      f32x4_t s0 = f32x4_t{0.f, 0.f, 0.f, 0.f}, s1 = s0;
      const uint16_t* r0 = &s_rows[rs][c][8 * g];
      const uint16_t* r1 = &s_rows[rs][16 + c][8 * g];
#pragma unroll
      for (int kb = 0; kb < KS; ++kb) {
        s0 = mfma_bf16_16x16x32(*reinterpret_cast<const u32x4_t*>(r0 + 32 * kb), qb[kb], s0);
        s1 = mfma_bf16_16x16x32(*reinterpret_cast<const u32x4_t*>(r1 + 32 * kb), qb[kb], s1);
      }
      float p[8];
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float x0 = (s_info[rs][4 * g + r] & 1) ? s0[r] * a.scale_log2 : -INFINITY;
        const float x1 = (s_info[rs][16 + 4 * g + r] & 1) ? s1[r] * a.scale_log2 : -INFINITY;
        p[r] = x0;
        p[4 + r] = x1;
        mx = fmaxf(mx, fmaxf(x0, x1));
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const bool none = m_new == -INFINITY;
      const float alpha = none ? 1.f : exp2f(m_run - m_new);
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        p[i] = none ? 0.f : exp2f(p[i] - m_new);
        psum += p[i];
      }
      l_run = l_run * alpha + psum;
      m_run = m_new;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) o[i][e] *= alpha;
      u32x4_t pb;
      pb[0] = pack_bf16_rne(p[0], p[1]);
      pb[1] = pack_bf16_rne(p[2], p[3]);
      pb[2] = pack_bf16_rne(p[4], p[5]);
      pb[3] = pack_bf16_rne(p[6], p[7]);
#pragma unroll
      for (int gd = 0; gd < 4; ++gd) {
        u32x4_t vr[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          vr[j] = *reinterpret_cast<const u32x4_t*>(&s_rows[rs][4 * g + j][128 * gd + 8 * c]);
          vr[4 + j] = *reinterpret_cast<const u32x4_t*>(&s_rows[rs][16 + 4 * g + j][128 * gd + 8 * c]);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int w = e >> 1;
          const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
          u32x4_t av;
#pragma unroll
          for (int pp = 0; pp < 4; ++pp) av[pp] = __builtin_amdgcn_perm(vr[2 * pp + 1][w], vr[2 * pp][w], sel);
          o[gd][e] = mfma_bf16_16x16x32(av, pb, o[gd][e]);
        }
      }
    }
    __syncthreads();
  }

  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);

  // ---- merge the row streams of each head tile (LDS, reusing the row buffers)
  if constexpr (RS > 1) {
    constexpr int STRIDE = 4 * 8 * 4 * 64 + 32;
    static_assert((RS - 1) * HT * STRIDE * 4 <= (int)sizeof(s_rows), "merge scratch");
    float* scratch = reinterpret_cast<float*>(&s_rows[0][0][0]);
    if (rs > 0) {
      float* dst = scratch + ((rs - 1) * HT + ht) * STRIDE;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e)
#pragma unroll
          for (int r = 0; r < 4; ++r) dst[((i * 8 + e) * 4 + r) * 64 + lane] = o[i][e][r];
      if (g == 0) {
        dst[8192 + c] = m_run;
        dst[8192 + 16 + c] = l_run;
      }
    }
    __syncthreads();
    if (rs == 0) {
#pragma unroll 1
      for (int q = 1; q < RS; ++q) {
        const float* src = scratch + ((q - 1) * HT + ht) * STRIDE;
        const float mq = src[8192 + c];
        const float lq = src[8192 + 16 + c];
        const float m_new = fmaxf(m_run, mq);
        const bool none = m_new == -INFINITY;
        const float a0 = none ? 0.f : exp2f(m_run - m_new);
        const float aq = none ? 0.f : exp2f(mq - m_new);
        l_run = l_run * a0 + lq * aq;
        m_run = m_new;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int e = 0; e < 8; ++e)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              o[i][e][r] = o[i][e][r] * a0 + src[((i * 8 + e) * 4 + r) * 64 + lane] * aq;
      }
    }
  }

  const int head = head0 + c;
  if constexpr (!SPLIT) {
    if (rs == 0) {
      const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
      uint16_t* op = a.out + (int64_t)t * a.ld_out + (int64_t)head * kDV;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          u32x4_t v;
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2)
            v[e2] = pack_bf16_rne(o[i][2 * e2][r] * inv, o[i][2 * e2 + 1][r] * inv);
          *reinterpret_cast<u32x4_t*>(op + 128 * i + 32 * g + 8 * r) = v;
        }
      if (a.lse && g == 0)
        a.lse[(int64_t)t * a.H + head] = l_run > 0.f ? (m_run + __log2f(l_run)) * kLn2 : -INFINITY;
    }
  } else {
    if (rs == 0) {
      float* po = a.part_o + (((int64_t)t * a.H + head) * a.n_split + split) * kDV;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          f32x4_t v0, v1;
#pragma unroll
          for (int e = 0; e < 4; ++e) { v0[e] = o[i][e][r]; v1[e] = o[i][4 + e][r]; }
          float* d = po + 128 * i + 32 * g + 8 * r;
          *reinterpret_cast<f32x4_t*>(d) = v0;
          *reinterpret_cast<f32x4_t*>(d + 4) = v1;
        }
      if (g == 0) {
        float* pml = a.part_ml + (((int64_t)t * a.H + head) * a.n_split + split) * 2;
        pml[0] = m_run;
        pml[1] = l_run;
      }
    }
    // last workgroup of this (row, head group) merges the splits
    __threadfence();
    __syncthreads();
    uint32_t* ctr = a.counters + (int64_t)t * gridDim.y + hg;
    if (threadIdx.x == 0) s_flag = (atomicAdd(ctr, 1u) == (uint32_t)a.n_split - 1) ? 1u : 0u;
    __syncthreads();
    if (!s_flag) return;
    __threadfence();
    constexpr int NH = HT * 16;
    // 256 threads: 16 per head, each 32 consecutive columns
    for (int hh = threadIdx.x / 16; hh < NH; hh += 16) {
      const int hd = hg * NH + hh;
      const int d0 = (threadIdx.x % 16) * 32;
      const float* pml = a.part_ml + ((int64_t)t * a.H + hd) * a.n_split * 2;
      const float* po = a.part_o + ((int64_t)t * a.H + hd) * a.n_split * kDV + d0;
      float ms = -INFINITY;
      for (int s = 0; s < a.n_split; ++s) ms = fmaxf(ms, pml[2 * s]);
      float acc[32];
#pragma unroll
      for (int d = 0; d < 32; ++d) acc[d] = 0.f;
      float ls = 0.f;
      if (ms != -INFINITY) {
        for (int s = 0; s < a.n_split; ++s) {
          const float wgt = exp2f(pml[2 * s] - ms);
          ls += wgt * pml[2 * s + 1];
          const f32x4_t* src = reinterpret_cast<const f32x4_t*>(po + (int64_t)s * kDV);
#pragma unroll
          for (int d = 0; d < 8; ++d) {
            const f32x4_t v = src[d];
            acc[4 * d] += wgt * v[0];
            acc[4 * d + 1] += wgt * v[1];
            acc[4 * d + 2] += wgt * v[2];
            acc[4 * d + 3] += wgt * v[3];
          }
        }
      }
      const float inv = ls > 0.f ? 1.f / ls : 0.f;
      uint16_t* op = a.out + (int64_t)t * a.ld_out + (int64_t)hd * kDV + d0;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        u32x4_t v;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2)
          v[e2] = pack_bf16_rne(acc[8 * d + 2 * e2] * inv, acc[8 * d + 2 * e2 + 1] * inv);
        *reinterpret_cast<u32x4_t*>(op + 8 * d) = v;
      }
      if (a.lse && (threadIdx.x % 16) == 0)
        a.lse[(int64_t)t * a.H + hd] = ls > 0.f ? (ms + __log2f(ls)) * kLn2 : -INFINITY;
    }
    if (threadIdx.x == 0) *ctr = 0u;
  }
}

template <int FMT, int DQK, int HT>
static hipError_t launch_h(const MlaArgs& a, int T, hipStream_t st) {
  dim3 grid(a.n_split, a.H / (16 * HT), T);
  if (a.n_split > 1)
    hipLaunchKernelGGL((k_sparse_mla<FMT, DQK, HT, true>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((k_sparse_mla<FMT, DQK, HT, false>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int FMT, int DQK>
static hipError_t launch_d(const MlaArgs& a, int ht, int T, hipStream_t st) {
  if (ht == 4) return launch_h<FMT, DQK, 4>(a, T, st);
  if (ht == 2) return launch_h<FMT, DQK, 2>(a, T, st);
  return launch_h<FMT, DQK, 1>(a, T, st);
}

hipError_t launch_sparse_mla(const MlaArgs& a, int fmt, int d_qk, int ht, int T, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  if (fmt == kFmtBf16) {
    if (d_qk == 576) return launch_d<kFmtBf16, 576>(a, ht, T, st);
    return launch_d<kFmtBf16, 512>(a, ht, T, st);
  }
  if (fmt == kFmtUniform) {
    if (d_qk == 576) return launch_d<kFmtUniform, 576>(a, ht, T, st);
    return launch_d<kFmtUniform, 512>(a, ht, T, st);
  }
  return launch_d<kFmtDsMla, 512>(a, ht, T, st);
}

}  // namespace dsa
