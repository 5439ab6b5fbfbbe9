// Backward of the sparse absorbed-MLA attention (one list, bf16 latent rows), gfx950 MFMA.
//
// For the forward out[t,h] = sum_i p_i c_i[0:d_v], p_i = exp(l_i - lse[t,h]),
// l_i = softmax_scale * q[t,h] . c_i[0:d_qk] over the listed rows c_i (entries -1 contribute
// nothing), an upstream gradient dout gives, with D = dout[t,h] . out[t,h]:
//   dl_i = p_i (dout[t,h] . c_i[0:d_v] - D)
//   dq[t,h] = softmax_scale * sum_i dl_i c_i[0:d_qk]
//   dkv[slot_i] += softmax_scale * dl_i q[t,h]  (columns 0:d_qk)  +  p_i dout[t,h]  (0:d_v)
//   dsink[h] += -exp(sink[h] - lse[t,h]) D
// (radixark/miles PR 3608, section "What": the backward takes the forward's lse with the sink
// folded in, and adds dKV through the listed indices atomically; the lse here may be in base 2).
//
// A workgroup takes one query row and 16 heads (4 waves), or 32 heads as two such groups of 4
// waves sharing the gathered rows (when dZ and P go to the workspace), and walks the row's list
// in blocks of 32 rows gathered into LDS (direct global->LDS loads). Per block, with S^T = K Q^T and
// dP^T = V dO^T split over the waves as in the forward (two row tiles x two halves of the
// contraction, the partials meeting in LDS):
//   * P and dZ from the forward's lse (no second pass over the list);
//   * dq^T += K^T dZ^T, with dZ^T taken straight from the S^T accumulator layout as the B
//     operand and K^T from an 8x8 transpose of LDS rows in registers (the forward's value
//     product); each wave owns 128 columns, the 64 RoPE columns are shared out in pairs of
//     column phases;
//   * scale dZ and P cross lanes once through LDS and go to a workspace as bf16 [row][head],
//     with the rows' resolved slots.
// A second kernel (k_sparse_mla_bwd_dkv) then forms dKV = (scale dZ)^T Q + P^T dO over ALL
// heads of a query row at once (32x32x8 MFMAs, k = heads; q and dout are its B operands, held
// in registers for the workgroup's column tiles), so that a listed row costs one fp32 atomic
// add per column whatever the head count: the atomics bound the backward, and summing the
// heads first divides them by H / 16. An atomic instruction covers 32 consecutive columns of
// 2 rows; rows of padding entries are skipped. With 16 heads there is nothing to sum first, and
// the first kernel adds dKV itself (same products, no workspace round trip).
// A cache row that exactly one list entry names (over all rows of the call) needs no atomic:
// with an owner map (one word per slot, marked by k_sparse_mla_bwd_mid: the first entry's
// row + 1 where the word was 0, bit 31 from every other entry and wherever it was not 0),
// k_sparse_mla_bwd_dkv_rows (32 or 64 padded heads) adds into such rows with plain loads and
// stores of whole cache rows, and keeps atomics for rows that several entries name. fp32
// atomics run at about one per L2 channel and clock; decode-shaped lists (each row its own
// request) name every row once. Without the map (or with 128 padded heads) every add is
// atomic (k_sparse_mla_bwd_dkv).
// Blocks stream through a ring of two: the next block's rows are requested before the
// current block's products (one workgroup per CU: nothing else hides a block's gather).
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace dsa {

namespace {

constexpr int kBwdNB = 32;         // rows per block
constexpr int kBwdResolve = 1024;  // list entries resolved to slots per pass
constexpr int kBwdDV = 512;

typedef __attribute__((ext_vector_type(4))) short s16x4_t;

// 16x16x16 bf16 MFMA: lane l supplies A[l%16][4(l/16)+j] and B[4(l/16)+j][l%16] (j = 0..3)
// and receives C[4(l/16)+r][l%16] (r = 0..3).
__device__ __forceinline__ f32x4_t mfma_bf16_16x16x16(u32x2_t a, u32x2_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, a),
                                                   __builtin_bit_cast(s16x4_t, b), c, 0, 0, 0);
}

// 32x32x8 bf16 MFMA: lane l supplies A[l%32][4(l/32)+j] and B[4(l/32)+j][l%32] (j = 0..3) and
// receives C[8(r/4) + 4(l/32) + r%4][l%32] in accumulator r = 0..15.
__device__ __forceinline__ f32x16_t mfma_bf16_32x32x8(u32x2_t a, u32x2_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(__builtin_bit_cast(s16x4_t, a),
                                                  __builtin_bit_cast(s16x4_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t lds_u16(const uint16_t* p) { return *p; }

}  // namespace

// FUSED: dKV of the workgroup's 16 heads added straight from this kernel (a single 16-head group
// per row: nothing to sum first); else dZ and P go to the workspace for k_sparse_mla_bwd_dkv.
template <int DQK, bool FUSED>
__global__ __launch_bounds__(FUSED ? 256 : 512, 1) void k_sparse_mla_bwd(MlaBwdArgs a) {
  // 16-head groups per workgroup: two (8 waves) share the gathered rows when dZ and P go to
  // the workspace, one with the fused dKV
  constexpr int GRP = FUSED ? 1 : 2;
  constexpr int NW = 4 * GRP;
  constexpr int NT = 256 * GRP;
  // padded bf16 row in LDS, chunks swizzled by row_swz: the score and dP products' reads (16
  // rows at one 16-byte column) and the dq product's (256 bytes of rows 4 apart) are free of
  // bank conflicts (with 8 elements of padding and no swizzle they cost 4 cycles each)
  constexpr int RE = DQK + 32;
  static_assert((RE * 2) % 128 == 64, "row stride");
  constexpr int KS = DQK / 32;                // k-steps of the score product
  constexpr int KQ = KS / 2;                  // per wave (split over the two halves)
  constexpr bool kRope = DQK > kBwdDV;        // columns 512..575 (4 x 16) beyond the value
  constexpr int CT = DQK / 32;                // 32-column tiles of dKV
  constexpr int CTW = FUSED ? (CT + NW - 1) / NW : 1;   // per wave, at most
  static_assert(KS % 2 == 0, "shapes");
  __shared__ __align__(16) uint16_t s_rows[2][kBwdNB][RE];
  __shared__ __align__(16) int32_t s_slot[kBwdResolve];
  __shared__ const uint8_t* s_ra[kBwdNB];
  __shared__ f32x4_t s_ss[GRP][4][64];
  __shared__ f32x4_t s_sd[GRP][4][64];
  __shared__ __align__(16) uint16_t s_tz[GRP][kBwdNB][16];   // bf16 scale * dZ[row][head]
  __shared__ __align__(16) uint16_t s_tp[GRP][kBwdNB][16];   // bf16 P[row][head]
  __shared__ float s_D[GRP][16];
  __shared__ float s_l2[GRP][16];

  const int t = blockIdx.y;
  const int hg = blockIdx.x;
  const int sp = blockIdx.z;                  // part of the row's list
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int gi = wave >> 2;                   // head group of this wave
  const int lw = wave & 3;                    // wave within its group
  const int tg = threadIdx.x & 255;           // thread within its group
  const int g = lane >> 4;
  const int c = lane & 15;
  const int head0 = (hg * GRP + gi) * 16;
  const int b = min(max(a.row_req ? a.row_req[t] : t, 0), a.n_req - 1);
  const KvDev kv = a.kv;
  // the paging rebuilt field by field: a table/base select on the argument copy itself would
  // be lowered to an indexed load from a scratch copy of the struct
  const Paging pg = pick_paging(false, a.kv.pg, a.kv.pg);
  const int32_t* const idx = a.idx + (int64_t)t * a.ld_idx;
  const int ntot = a.n_idx;
  // this workgroup's entries [e0, e1): whole blocks of the list, part sp of gridDim.z
  const int eper = ((ntot + (int)gridDim.z - 1) / (int)gridDim.z + kBwdNB - 1) / kBwdNB * kBwdNB;
  const int e0 = min(ntot, sp * eper);
  const int e1 = min(ntot, e0 + eper);

  // ---- prologue: q and dout of the 16 heads staged in the row buffer, the register operands
  // built from them; D = dout . out and the lse in base 2 per head
  constexpr int DOS = kBwdDV + 16;           // padded like the rows
  static_assert(GRP * (16 * RE + 16 * DOS) <= 2 * kBwdNB * RE, "staging");
  uint16_t* const s_q = &s_rows[0][0][0] + gi * (16 * RE + 16 * DOS);   // [16][RE]
  uint16_t* const s_do = s_q + 16 * RE;                                  // [16][DOS]
  // Heads past H (a head count that is not a whole number of 16-head groups) read q, dout and
  // out as zero and lse as 0: their P is finite and their dZ and P dout are zero, so they add
  // nothing to dKV, and nothing of them is written.
  // valid heads of this group (<= 0: a group of padding heads only, with two groups per
  // workgroup); every read below takes a head of the row (min(head, H - 1)) and drops it
  const int hval = a.H - head0;
  {
    // q and dout of the group (its 256 threads): every 16-byte load of the thread requested at
    // once, then stored (a loop of load, wait, store pays a round trip each)
    const uint16_t* qr = a.q + (int64_t)t * a.ld_q;
    const uint16_t* dr = a.dout + (int64_t)t * a.ld_dout;
    constexpr int NTG = 256;
    constexpr int NQ = (16 * DQK / 8 + NTG - 1) / NTG;
    constexpr int ND = 16 * kBwdDV / 8 / NTG;
    static_assert(16 * kBwdDV % (8 * NTG) == 0, "whole dout loads");
    u32x4_t vq[NQ], vd[ND];
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      const int o = min((tg + j * NTG) * 8, 16 * DQK - 8);
      vq[j] = *reinterpret_cast<const u32x4_t*>(qr + (int64_t)min(head0 + o / DQK, a.H - 1) * DQK + o % DQK);
    }
#pragma unroll
    for (int j = 0; j < ND; ++j) {
      const int o = (tg + j * NTG) * 8;
      vd[j] = *reinterpret_cast<const u32x4_t*>(dr + (int64_t)min(head0 + o / kBwdDV, a.H - 1) * kBwdDV + o % kBwdDV);
    }
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      const int o = (tg + j * NTG) * 8;
      if (o < 16 * DQK)
        *reinterpret_cast<u32x4_t*>(s_q + (o / DQK) * RE + o % DQK) = o / DQK < hval ? vq[j] : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < ND; ++j) {
      const int o = (tg + j * NTG) * 8;
      *reinterpret_cast<u32x4_t*>(s_do + (o / kBwdDV) * DOS + o % kBwdDV) = o / kBwdDV < hval ? vd[j] : u32x4_t{0u, 0u, 0u, 0u};
    }
    // D: 16 threads per head, 32 columns each
    const int h = tg >> 4;
    const int c0 = (tg & 15) * 32;
    const int hr = min(head0 + h, a.H - 1);             // padding heads read a valid row, then drop it
    const uint16_t* og = a.out + (int64_t)t * a.ld_out + (int64_t)hr * kBwdDV + c0;
    const uint16_t* dh = dr + (int64_t)hr * kBwdDV + c0;
    float d = 0.f;
#pragma unroll
    for (int i = 0; i < 32; i += 8) {
      const u32x4_t ov = *reinterpret_cast<const u32x4_t*>(og + i);
      const u32x4_t dv = *reinterpret_cast<const u32x4_t*>(dh + i);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        d = fmaf(__uint_as_float(ov[j] << 16), __uint_as_float(dv[j] << 16), d);
        d = fmaf(__uint_as_float(ov[j] & 0xffff0000u), __uint_as_float(dv[j] & 0xffff0000u), d);
      }
    }
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) d += __shfl_xor(d, m);
    if ((tg & 15) == 0) {
      s_D[gi][h] = h < hval ? d : 0.f;
      const float l = h < hval ? a.lse[(int64_t)t * a.H + head0 + h] : 0.f;
      s_l2[gi][h] = a.lse_log2 ? l : l * kLog2e;
    }
  }
  __syncthreads();
  // B operand of S^T = K Q^T for this wave's half of the contraction, and of dP^T = V dO^T
  const int kq0 = (lw & 1) * KQ;
  u32x4_t qb[KQ];
#pragma unroll
  for (int kb = 0; kb < KQ; ++kb) qb[kb] = *reinterpret_cast<const u32x4_t*>(s_q + c * RE + 32 * (kq0 + kb) + 8 * g);
  u32x4_t dob[8];
#pragma unroll
  for (int kb = 0; kb < 8; ++kb)
    dob[kb] = *reinterpret_cast<const u32x4_t*>(s_do + c * DOS + 256 * (lw & 1) + 32 * kb + 8 * g);
  // B operands of dKV (k = the 16 heads in two steps of 8, n = 32 columns): Q and dO for the
  // wave's column tiles ct0 .. ct0 + nct - 1 (tile counts (CT + 3 - w) / 4: 5, 5, 4, 4 of 18)
  const int nct = (CT + NW - 1 - wave) / NW;
  const int ct0 = wave * (CT / NW) + min(wave, CT % NW);
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  u32x2_t qkb[CTW][2], dkb[CTW][2];
#pragma unroll
  for (int k = 0; k < CTW; ++k) {
    if constexpr (!FUSED) break;
    const int col = min(ct0 + k, CT - 1) * 32 + l32;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      uint32_t h4[4], d4[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int head = 8 * ks + 4 * hh + j;
        h4[j] = lds_u16(s_q + head * RE + col);
        d4[j] = col < kBwdDV ? lds_u16(s_do + head * DOS + col) : 0u;
      }
      qkb[k][ks] = u32x2_t{h4[0] | (h4[1] << 16), h4[2] | (h4[3] << 16)};
      dkb[k][ks] = u32x2_t{d4[0] | (d4[1] << 16), d4[2] | (d4[3] << 16)};
    }
  }
  const float Dc = s_D[gi][c];
  const float l2c = s_l2[gi][c];
  if (sp == 0 && a.sink && a.dsink && tg < min(16, hval)) {
    const float sk = a.sink[head0 + tg];
    if (sk > -INFINITY) unsafeAtomicAdd(a.dsink + head0 + tg, -exp2f(sk * kLog2e - s_l2[gi][tg]) * s_D[gi][tg]);
  }
  __syncthreads();   // the staging area becomes the row buffer

  // dq^T accumulators: 128 columns of group `lw` (8 column phases), and for d_qk = 576 two
  // phases of the RoPE group (columns 512 + 8 m + e, e = 2 lw + i, m < 8)
  f32x4_t oq[8];
  f32x4_t o4[2];
#pragma unroll
  for (int e = 0; e < 8; ++e) oq[e] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  o4[0] = o4[1] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  int pass_n = 0;
  for (int p0 = e0; p0 < e1; p0 += kBwdResolve) {
    const int p1 = min(e1, p0 + kBwdResolve);
    const int nb = (p1 - p0 + kBwdNB - 1) / kBwdNB;
    pass_n = p1 - p0;
    {   // the pass's entries to slots: every index read, then every table read
      constexpr int RPT = kBwdResolve / NT;
      int e[RPT];
#pragma unroll
      for (int k = 0; k < RPT; ++k) e[k] = idx[min(p0 + (int)threadIdx.x + k * NT, p1 - 1)];
      SlotRead sr[RPT];
#pragma unroll
      for (int k = 0; k < RPT; ++k) sr[k] = slot_read(pg, b, max(e[k], 0));
#pragma unroll
      for (int k = 0; k < RPT; ++k) {
        const int j = threadIdx.x + k * NT;
        const int64_t sl = slot_done(pg, sr[k]);
        if (j < pass_n) s_slot[j] = e[k] >= 0 ? (int32_t)sl : -1;
      }
    }
    __syncthreads();
    // row addresses of block ib (one lane per row; padding reads row 0)
    auto row_addrs = [&](int ib) {
      if (threadIdx.x < kBwdNB) {
        const int j = ib * kBwdNB + threadIdx.x;
        const int32_t v = j < pass_n ? s_slot[j] : -1;
        s_ra[threadIdx.x] = kv.data + (int64_t)max(v, 0) * (DQK * 2);
      }
    };
    // that block's loads into ring buffer buf (addresses in s_ra)
    auto gather = [&](int buf) {
      constexpr int RW = RE / 8;                   // 16-byte slots per padded row
      constexpr int SLOTS = kBwdNB * RW;
      constexpr int NINS = (SLOTS + 63) / 64;
      constexpr int PER = (NINS + NW - 1) / NW;
      auto* lbase = reinterpret_cast<__attribute__((address_space(3))) uint8_t*>(
          reinterpret_cast<uintptr_t>(&s_rows[buf][0][0]) & 0xffffffffu);
      const uint8_t* src[PER];
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        const int j = min((wave + k * NW) * 64 + lane, SLOTS - 1);
        const int r = j / RW;
        int cc = j - r * RW;
        cc = cc >= DQK / 8 ? cc - DQK / 8 : cc ^ row_swz(r);   // pad slots: the row's start
        src[k] = s_ra[r] + 16 * cc;
      }
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        const int ins = wave + k * NW;
        if (ins < NINS && ins * 64 + lane < SLOTS) {
          const uint8_t* sp = src[k];
          __builtin_amdgcn_global_load_lds(sp, lbase + ins * 1024, 16, 0, 0);
        }
      }
    };
    row_addrs(0);
    lds_barrier();
    gather(0);
    for (int it = 0; it < nb; ++it) {
      const int jb = it * kBwdNB;
      const int cur = it & 1;
      // this block's rows are in (and every vector-memory operation of the previous block is
      // done); the next block's addresses (every wave is done with the previous ones: the
      // products below pass barriers), then its loads, which land while this block is used
      wait_vmcnt<0>();
      if (it + 1 < nb) row_addrs(it + 1);
      lds_barrier();
      if (it + 1 < nb) gather(cur ^ 1);           // that buffer held block it - 1

      // ---- S^T and dP^T, split over the waves
      const int jm = jb + 4 * g;
      const u32x4_t sl0 = *reinterpret_cast<const u32x4_t*>(&s_slot[jm]);
      const u32x4_t sl1 = *reinterpret_cast<const u32x4_t*>(&s_slot[jm + 16]);
      {
        const uint16_t* rp = &s_rows[cur][16 * (lw >> 1) + c][8 * (g ^ row_swz(c))];
        f32x4_t sp = f32x4_t{0.f, 0.f, 0.f, 0.f}, dp = sp;
#pragma unroll
        for (int kb = 0; kb < KQ; ++kb)
          sp = mfma_bf16_16x16x32(*reinterpret_cast<const u32x4_t*>(rp + 32 * (kq0 + kb)), qb[kb], sp);
#pragma unroll
        for (int kb = 0; kb < 8; ++kb)
          dp = mfma_bf16_16x16x32(*reinterpret_cast<const u32x4_t*>(rp + 256 * (lw & 1) + 32 * kb), dob[kb], dp);
        s_ss[gi][lw][lane] = sp;
        s_sd[gi][lw][lane] = dp;
      }
      lds_barrier();
      const f32x4_t s0 = s_ss[gi][0][lane] + s_ss[gi][1][lane], s1 = s_ss[gi][2][lane] + s_ss[gi][3][lane];
      const f32x4_t d0 = s_sd[gi][0][lane] + s_sd[gi][1][lane], d1 = s_sd[gi][2][lane] + s_sd[gi][3][lane];
      // ---- P and dZ of rows 4g + r and 16 + 4g + r, head c
      float p[8], dz[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool ok0 = jm + r < pass_n && (int32_t)sl0[r] >= 0;
        const bool ok1 = jm + 16 + r < pass_n && (int32_t)sl1[r] >= 0;
        p[r] = ok0 ? exp2_hw(s0[r] * a.scale_log2 - l2c) : 0.f;
        p[4 + r] = ok1 ? exp2_hw(s1[r] * a.scale_log2 - l2c) : 0.f;
        dz[r] = p[r] * (d0[r] - Dc);
        dz[4 + r] = p[4 + r] * (d1[r] - Dc);
      }
      // dZ and P into LDS, row-major by head, for the dKV product's B layout
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        s_tz[gi][4 * g + r][c] = (uint16_t)bf16_rne_bits(dz[r] * a.scale);
        s_tz[gi][16 + 4 * g + r][c] = (uint16_t)bf16_rne_bits(dz[4 + r] * a.scale);
        s_tp[gi][4 * g + r][c] = (uint16_t)bf16_rne_bits(p[r]);
        s_tp[gi][16 + 4 * g + r][c] = (uint16_t)bf16_rne_bits(p[4 + r]);
      }
      if constexpr (!FUSED) {
        // every wave's dZ and P in LDS; they go out before the dq product, so that the stores
        // have its time to complete before the next block's wait
        lds_barrier();
        // ---- scale dZ, P (bf16, [row][head] with the row's heads contiguous) and the slots to
        // the workspace for the dKV kernel: 16 bytes (8 heads) per thread
        if (tg < 2 * 2 * kBwdNB) {
          const int arr = tg >> 6;                       // 0: dZ, 1: P
          const int row = (tg >> 1) & (kBwdNB - 1);
          const int half = tg & 1;
          const int j = jb + row;
          if (j < pass_n) {
            const uint16_t* src = arr ? &s_tp[gi][row][8 * half] : &s_tz[gi][row][8 * half];
            uint16_t* dst = (arr ? a.ws_p : a.ws_dz) + ((int64_t)t * ntot + p0 + j) * a.Hp + head0 + 8 * half;
            *reinterpret_cast<u32x4_t*>(dst) = *reinterpret_cast<const u32x4_t*>(src);
          }
        }
        if (hg == 0 && threadIdx.x < kBwdNB && jb + (int)threadIdx.x < pass_n)
          a.ws_slot[(int64_t)t * ntot + p0 + jb + threadIdx.x] = s_slot[jb + threadIdx.x];
      }
      // ---- dq^T += K^T dZ^T: dZ^T from the accumulator layout (k-slot 8g + i of the B
      // operand is row 4g + i, then 16 + 4g + i - 4), K^T by 8x8 transposes of LDS rows
      u32x4_t zb;
      zb[0] = pack_bf16_rne(dz[0], dz[1]);
      zb[1] = pack_bf16_rne(dz[2], dz[3]);
      zb[2] = pack_bf16_rne(dz[4], dz[5]);
      zb[3] = pack_bf16_rne(dz[6], dz[7]);
      {
        u32x4_t vr[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          vr[j] = *reinterpret_cast<const u32x4_t*>(&s_rows[cur][4 * g + j][128 * lw + 8 * (c ^ row_swz(4 * g))]);
          vr[4 + j] = *reinterpret_cast<const u32x4_t*>(&s_rows[cur][16 + 4 * g + j][128 * lw + 8 * (c ^ row_swz(4 * g))]);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int w = e >> 1;
          const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
          u32x4_t av;
#pragma unroll
          for (int pp = 0; pp < 4; ++pp) av[pp] = __builtin_amdgcn_perm(vr[2 * pp + 1][w], vr[2 * pp][w], sel);
          oq[e] = mfma_bf16_16x16x32(av, zb, oq[e]);
        }
      }
      if constexpr (kRope) {   // columns 512 + 8 m + e for m = c < 8; phases e = 2 lw + i
        // (the two phases of a wave are the two halves of dword `lw` of the 8 columns)
        uint32_t vw[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          vw[j] = *reinterpret_cast<const uint32_t*>(&s_rows[cur][4 * g + j][kBwdDV + 8 * ((c & 7) ^ row_swz(4 * g)) + 2 * lw]);
          vw[4 + j] = *reinterpret_cast<const uint32_t*>(&s_rows[cur][16 + 4 * g + j][kBwdDV + 8 * ((c & 7) ^ row_swz(4 * g)) + 2 * lw]);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const uint32_t sel = i ? 0x07060302u : 0x05040100u;
          u32x4_t av;
#pragma unroll
          for (int pp = 0; pp < 4; ++pp) av[pp] = c < 8 ? __builtin_amdgcn_perm(vw[2 * pp + 1], vw[2 * pp], sel) : 0u;
          o4[i] = mfma_bf16_16x16x32(av, zb, o4[i]);
        }
      }
      if constexpr (FUSED) {
        lds_barrier();
        // ---- dKV = (scale dZ)^T Q + P^T dO over the 16 heads (m = the 32 rows, n = 32 columns):
        // accumulator r of lane l is row 8 (r / 4) + 4 hh + r % 4 and column tile * 32 + l32
        u32x2_t az[2], ap[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          az[ks] = *reinterpret_cast<const u32x2_t*>(&s_tz[gi][l32][8 * ks + 4 * hh]);
          ap[ks] = *reinterpret_cast<const u32x2_t*>(&s_tp[gi][l32][8 * ks + 4 * hh]);
        }
        int32_t rs[16];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int r0 = 8 * q4 + 4 * hh;
          const u32x4_t sv = *reinterpret_cast<const u32x4_t*>(&s_slot[jb + r0]);
#pragma unroll
          for (int i = 0; i < 4; ++i) rs[4 * q4 + i] = jb + r0 + i < pass_n ? (int32_t)sv[i] : -1;
        }
#pragma unroll
        for (int k = 0; k < CTW; ++k) {
          if (k < nct) {
            const int col = (ct0 + k) * 32 + l32;
            f32x16_t acc = {};
            acc = mfma_bf16_32x32x8(az[0], qkb[k][0], acc);
            acc = mfma_bf16_32x32x8(az[1], qkb[k][1], acc);
            if ((ct0 + k) * 32 < kBwdDV) {
              acc = mfma_bf16_32x32x8(ap[0], dkb[k][0], acc);
              acc = mfma_bf16_32x32x8(ap[1], dkb[k][1], acc);
            }
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (rs[r] >= 0) unsafeAtomicAdd(a.dkv + (int64_t)rs[r] * DQK + col, acc[r]);
          }
        }
      }
    }
    __syncthreads();   // every wave is done with this pass's slots
  }

  // ---- dq: lane (c = head, g) holds columns 128 lw + 8 (4g + r) + e (and the RoPE phases);
  // the list's first part writes dq, the others their partial sums for the next kernel to add
  if (c >= hval) return;                                // a padding head: no dq
  float* dqh = sp == 0 ? a.dq + (int64_t)t * a.ld_dq + (int64_t)(head0 + c) * DQK
                       : a.ws_dqp + (((int64_t)(sp - 1) * gridDim.y + t) * a.H + head0 + c) * DQK;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    f32x4_t v0, v1;
#pragma unroll
    for (int e = 0; e < 4; ++e) { v0[e] = oq[e][r] * a.scale; v1[e] = oq[4 + e][r] * a.scale; }
    float* d = dqh + 128 * lw + 8 * (4 * g + r);
    *reinterpret_cast<f32x4_t*>(d) = v0;
    *reinterpret_cast<f32x4_t*>(d + 4) = v1;
  }
  if constexpr (kRope) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = 4 * g + r;
      if (m < 8) {
#pragma unroll
        for (int i = 0; i < 2; ++i) dqh[kBwdDV + 8 * m + 2 * lw + i] = o4[i][r] * a.scale;
      }
    }
  }
}

// dKV of one query row over all its heads, for CG 32-column tiles: workgroup (tile group, row),
// its 4 waves take every 4th 32-row block of the row's list. B operands (k = heads in steps of
// 8, n = 32 columns): q and dout of the row, built once; A operands: scale dZ and P of the
// block's 32 rows from the workspace (lane l: row l % 32, heads 8 ks + 4 (l / 32) .. + 3).
template <int DQK, int HK>   // HK = H / 8 head steps
__global__ __launch_bounds__(256, 1) void k_sparse_mla_bwd_dkv(MlaBwdArgs a, int cg) {
  constexpr int CT = DQK / 32;
  constexpr int CGM = HK >= 16 ? 2 : 3;       // tiles per workgroup, at most (registers)
  const int t = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int ct0 = blockIdx.x * cg;
  const int nct = min(cg, CT - ct0);
  const int ntot = a.n_idx;
  u32x2_t qkb[CGM][HK], dkb[CGM][HK];
  {
    const uint16_t* qr = a.q + (int64_t)t * a.ld_q;
    const uint16_t* dr = a.dout + (int64_t)t * a.ld_dout;
#pragma unroll
    for (int k = 0; k < CGM; ++k) {
      const int col = min(ct0 + k, CT - 1) * 32 + l32;
#pragma unroll
      for (int ks = 0; ks < HK; ++ks) {
        uint32_t h4[4], d4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int head = 8 * ks + 4 * hh + j;
          const bool hv = head < a.H;                   // padding heads: zero operands
          h4[j] = hv ? qr[(int64_t)head * DQK + col] : 0u;
          d4[j] = hv && col < kBwdDV ? dr[(int64_t)head * kBwdDV + col] : 0u;
        }
        qkb[k][ks] = u32x2_t{h4[0] | (h4[1] << 16), h4[2] | (h4[3] << 16)};
        dkb[k][ks] = u32x2_t{d4[0] | (d4[1] << 16), d4[2] | (d4[3] << 16)};
      }
    }
  }
  const int nb = (ntot + 31) / 32;
  for (int blk = wave; blk < nb; blk += 4) {
    const int r0 = blk * 32;
    // this lane's A rows and the slots of the 16 rows its accumulators hold
    const int ra = min(r0 + l32, ntot - 1);
    const uint16_t* zr = a.ws_dz + ((int64_t)t * ntot + ra) * a.Hp + 4 * hh;
    const uint16_t* pr = a.ws_p + ((int64_t)t * ntot + ra) * a.Hp + 4 * hh;
    u32x2_t az[HK], ap[HK];
#pragma unroll
    for (int ks = 0; ks < HK; ++ks) {
      az[ks] = *reinterpret_cast<const u32x2_t*>(zr + 8 * ks);
      ap[ks] = *reinterpret_cast<const u32x2_t*>(pr + 8 * ks);
    }
    int32_t rs[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = r0 + 8 * (r >> 2) + 4 * hh + (r & 3);
      rs[r] = row < ntot ? a.ws_slot[(int64_t)t * ntot + row] : -1;
    }
#pragma unroll
    for (int k = 0; k < CGM; ++k) {
      if (k < nct) {
        const int col = (ct0 + k) * 32 + l32;
        f32x16_t acc = {};
#pragma unroll
        for (int ks = 0; ks < HK; ++ks) acc = mfma_bf16_32x32x8(az[ks], qkb[k][ks], acc);
        if ((ct0 + k) * 32 < kBwdDV) {
#pragma unroll
          for (int ks = 0; ks < HK; ++ks) acc = mfma_bf16_32x32x8(ap[ks], dkb[k][ks], acc);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (rs[r] >= 0) unsafeAtomicAdd(a.dkv + (int64_t)rs[r] * DQK + col, acc[r]);
      }
    }
  }
}

// Between the backward's kernels, on one flat grid: blocks [0, nbm) mark the owner map (one
// thread per list entry, if there is a map); the rest add the dq partial sums of list parts
// 1..nsplit-1 into dq (one 16-byte piece per thread).
// The owner map: slot -> first naming row + 1, bit 31 when a second entry (of any row, or the
// same row again) names it. A word is positive afterwards only if it was 0 before and one
// entry alone names the slot: words that start dirty (a fresh workspace, or one whose layout
// moved) only send their rows to atomics. The dKV kernel clears every word it reads, so a map
// is clean again for the next call.
__global__ __launch_bounds__(256) void k_sparse_mla_bwd_mid(MlaBwdArgs a, int T, int d_qk, int nbm) {
  if ((int)blockIdx.x < nbm) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= (int64_t)T * a.n_idx) return;
    const int32_t s = a.ws_slot[e];
    if (s < 0) return;
    const int32_t old = atomicCAS(a.ws_owner + s, 0, (int32_t)(e / a.n_idx) + 1);
    if (old != 0) atomicOr(a.ws_owner + s, (int32_t)0x80000000);
    return;
  }
  const int64_t f = ((int64_t)blockIdx.x - nbm) * 256 + threadIdx.x;   // 16-byte piece of dq
  const int per_row = a.H * d_qk / 4;
  if (f >= (int64_t)T * per_row) return;
  const int t = (int)(f / per_row);
  const int o = (int)(f % per_row) * 4;
  f32x4_t v = *reinterpret_cast<const f32x4_t*>(a.dq + (int64_t)t * a.ld_dq + o);
  for (int k = 1; k < a.nsplit; ++k)
    v += *reinterpret_cast<const f32x4_t*>(a.ws_dqp + ((int64_t)(k - 1) * T + t) * a.H * d_qk + o);
  *reinterpret_cast<f32x4_t*>(a.dq + (int64_t)t * a.ld_dq + o) = v;
}

// dKV by whole cache rows (32 or 64 padded heads): a workgroup of 8 waves takes one query row
// and a run of its 32-entry blocks. Per block the scale dZ and P rows are staged in LDS once,
// each wave forms its column tiles (w, w + 8, w + 16) of the 32 x d_qk sums, the sums meet
// in LDS, and every thread then adds whole 16-byte pieces of the cache rows: each row's d_qk
// floats are read and written by one workgroup at once (the per-column-group kernel writes
// each row in 128-byte pieces from 9 workgroups, which keeps the HBM writes scattered).
// Rows named by this entry alone (owner map) take a plain load and store, rows named more
// than once atomics, padding nothing. The current values are requested before the products.
constexpr int kDkvBpwMax = 16;   // blocks per workgroup, at most

template <int DQK, int HK>
__global__ __launch_bounds__(512, 1) void k_sparse_mla_bwd_dkv_rows(MlaBwdArgs a, int bpw) {
  constexpr int NWV = 8;
  constexpr int CT = DQK / 32;                 // column tiles: 18 or 16
  constexpr int TPW = (CT + NWV - 1) / NWV;    // per wave, at most
  constexpr int HP = HK * 8;                   // padded heads of the workspace rows
  constexpr int ZS = HP + 4;                   // LDS row of dZ / P (bf16), 8-byte aligned
  constexpr int OS = DQK + 4;                  // LDS row of the sums (floats)
  constexpr int F4 = DQK / 4;                  // 16-byte pieces per cache row
  constexpr int NF = 32 * F4 / 512;            // pieces per thread and block
  static_assert(32 * F4 % 512 == 0, "whole pieces per thread");
  static_assert(HP % 8 == 0 && 32 * HP / 8 <= 256, "staging: one 16-byte piece per thread");
  __shared__ __align__(16) float s_out[32][OS];
  __shared__ __align__(16) uint16_t s_zp[2][32][ZS];
  __shared__ int32_t s_rs[kDkvBpwMax * 32];
  __shared__ uint32_t s_shared;                // bit b: block b0 + b has a row named more than once
  if (threadIdx.x == 0) s_shared = 0u;
  __syncthreads();
  const int t = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int ntot = a.n_idx;
  const int nbt = (ntot + 31) / 32;
  const int b0 = blockIdx.x * bpw;
  const int b1 = min(b0 + bpw, nbt);
  if (b0 >= b1) return;
  const int64_t rowe = (int64_t)t * ntot;      // this row's first workspace entry

  // the entries' slots and owner words, decoded into s_rs: >= 0 named by this entry alone,
  // -1 padding, <= -2 slot -(v + 2) named more than once
  static_assert(kDkvBpwMax * 32 % 512 == 0, "whole entries per thread");
  {
    constexpr int EPT = kDkvBpwMax * 32 / 512;
    int32_t v[EPT], o[EPT];
#pragma unroll
    for (int i = 0; i < EPT; ++i) v[i] = a.ws_slot[rowe + min(b0 * 32 + (int)threadIdx.x + 512 * i, ntot - 1)];
#pragma unroll
    for (int i = 0; i < EPT; ++i) o[i] = a.ws_owner ? a.ws_owner[max(v[i], 0)] : -1;
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      const int j = threadIdx.x + 512 * i;
      const bool mine = j < (b1 - b0) * 32 && b0 * 32 + j < ntot && v[i] >= 0;
      const int32_t d = !mine ? -1 : o[i] > 0 ? v[i] : -(v[i] + 2);
      if (j < (b1 - b0) * 32) {
        s_rs[j] = d;
        if (d <= -2) atomicOr(&s_shared, 1u << (j >> 5));   // the block has a row named twice
      }
      // the word back to 0 for the next call: a slot named once has no other reader, and
      // another reader of a shared slot that finds 0 takes the atomic path all the same
      if (mine && a.ws_owner) a.ws_owner[v[i]] = 0;
    }
  }
  // B operands of this wave's column tiles (k = heads in steps of 8, n = 32 columns): q, then
  // dout, of the row staged in the sums' LDS (whole 16-byte loads, padding heads zero) and
  // gathered from there once
  u32x2_t qkb[TPW][HK], dkb[TPW][HK];
  {
    uint16_t* const stg = reinterpret_cast<uint16_t*>(&s_out[0][0]);
    static_assert(HP * DQK * 2 <= 32 * OS * 4, "staging fits");
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int W = m == 0 ? DQK : kBwdDV;               // row width (bf16)
      const int RS = W;                                  // LDS row (bf16)
      const uint16_t* src = m == 0 ? a.q + (int64_t)t * a.ld_q : a.dout + (int64_t)t * a.ld_dout;
      const int n16 = HP * W / 8;                        // 16-byte pieces
      constexpr int MAXP = (HP * DQK / 8 + 511) / 512;
      u32x4_t v[MAXP];
#pragma unroll
      for (int i = 0; i < MAXP; ++i) {
        const int pc = min((int)threadIdx.x + 512 * i, n16 - 1);
        const int head = pc / (W / 8);
        v[i] = *reinterpret_cast<const u32x4_t*>(src + (int64_t)min(head, a.H - 1) * W + 8 * (pc % (W / 8)));
      }
#pragma unroll
      for (int i = 0; i < MAXP; ++i) {
        const int pc = threadIdx.x + 512 * i;
        const int head = pc / (W / 8);
        if (pc < n16)
          *reinterpret_cast<u32x4_t*>(stg + head * RS + 8 * (pc % (W / 8))) = head < a.H ? v[i] : u32x4_t{0u, 0u, 0u, 0u};
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < TPW; ++k) {
        const int col = min(wave + NWV * k, CT - 1) * 32 + l32;
#pragma unroll
        for (int ks = 0; ks < HK; ++ks) {
          uint32_t h4[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) h4[j] = col < W ? stg[(8 * ks + 4 * hh + j) * RS + col] : 0u;
          const u32x2_t b = u32x2_t{h4[0] | (h4[1] << 16), h4[2] | (h4[3] << 16)};
          if (m == 0) qkb[k][ks] = b;
          else dkb[k][ks] = b;
        }
      }
      __syncthreads();
    }
  }

  for (int blk = b0; blk < b1; ++blk) {
    const int jb = (blk - b0) * 32;
    // the current values of this thread's pieces of the block's rows (exclusively named rows;
    // other pieces read row 0 and drop it), and the block's dZ / P rows
    int32_t rsk[NF];
#pragma unroll
    for (int k = 0; k < NF; ++k) rsk[k] = s_rs[jb + ((int)threadIdx.x + 512 * k) / F4];
    f32x4_t cur[NF];
#pragma unroll
    for (int k = 0; k < NF; ++k)
      cur[k] = *reinterpret_cast<const f32x4_t*>(a.dkv + (int64_t)max(rsk[k], 0) * DQK + 4 * (((int)threadIdx.x + 512 * k) % F4));
    u32x4_t zp;
    const int zj = threadIdx.x & 255;                   // piece (row, 8 heads) of array zarr
    const int zarr = threadIdx.x >> 8;
    const int zrow = zj / (HP / 8);
    const int zpc = zj % (HP / 8);
    const bool zok = zj < 32 * HP / 8;
    {
      const int e = min(blk * 32 + zrow, ntot - 1);
      const uint16_t* src = (zarr ? a.ws_p : a.ws_dz) + (rowe + e) * a.Hp + 8 * zpc;
      zp = *reinterpret_cast<const u32x4_t*>(src);
    }
    if (zok) {   // two 8-byte stores: the padded LDS rows are 8-byte aligned, not 16
      uint16_t* zd = &s_zp[zarr][zrow][8 * zpc];
      reinterpret_cast<u32x2_t*>(zd)[0] = u32x2_t{zp[0], zp[1]};
      reinterpret_cast<u32x2_t*>(zd)[1] = u32x2_t{zp[2], zp[3]};
    }
    __syncthreads();                                    // staged; the last block's sums are read
    u32x2_t az[HK], ap[HK];
#pragma unroll
    for (int ks = 0; ks < HK; ++ks) {
      az[ks] = *reinterpret_cast<const u32x2_t*>(&s_zp[0][l32][8 * ks + 4 * hh]);
      ap[ks] = *reinterpret_cast<const u32x2_t*>(&s_zp[1][l32][8 * ks + 4 * hh]);
    }
#pragma unroll
    for (int k = 0; k < TPW; ++k) {
      const int ct = wave + NWV * k;
      if (ct < CT) {
        f32x16_t acc = {};
#pragma unroll
        for (int ks = 0; ks < HK; ++ks) acc = mfma_bf16_32x32x8(az[ks], qkb[k][ks], acc);
        if (ct * 32 < kBwdDV) {
#pragma unroll
          for (int ks = 0; ks < HK; ++ks) acc = mfma_bf16_32x32x8(ap[ks], dkb[k][ks], acc);
        }
        // accumulator r is row 8 (r / 4) + 4 hh + r % 4, column 32 ct + l32
#pragma unroll
        for (int r = 0; r < 16; ++r) s_out[8 * (r >> 2) + 4 * hh + (r & 3)][32 * ct + l32] = acc[r];
      }
    }
    __syncthreads();
    {
      f32x4_t v[NF];   // every sum of the thread read first (one LDS round trip), then stored
#pragma unroll
      for (int k = 0; k < NF; ++k) {
        const int f = threadIdx.x + 512 * k;
        v[k] = *reinterpret_cast<const f32x4_t*>(&s_out[f / F4][4 * (f % F4)]);
      }
#pragma unroll
      for (int k = 0; k < NF; ++k)
        if (rsk[k] >= 0)
          *reinterpret_cast<f32x4_t*>(a.dkv + (int64_t)rsk[k] * DQK + 4 * (((int)threadIdx.x + 512 * k) % F4)) = cur[k] + v[k];
    }
    // rows named more than once: atomics whose 64 lanes cover 64 consecutive floats (an atomic
    // instruction over 16-byte strided lanes costs the L2 about three times as much)
    if (s_shared >> (blk - b0) & 1u) {
#pragma unroll 1
      for (int k = 0; k < 4 * NF; ++k) {
        const int flat = 64 * ((int)(threadIdx.x >> 6) + 8 * k) + lane;
        const int r = flat / DQK;
        const int c = flat % DQK;
        const int32_t rs = s_rs[jb + r];
        if (rs <= -2) unsafeAtomicAdd(a.dkv + (int64_t)(-(rs + 2)) * DQK + c, s_out[r][c]);
      }
    }
  }
}

template <int DQK>
static void launch_dkv(const MlaBwdArgs& a, int T, hipStream_t st) {
  constexpr int CT = DQK / 32;
  const int hk = a.Hp / 8;
  if (hk <= 8 && a.ws_owner) {   // whole rows per workgroup (with the owner map)
    // blocks per workgroup: up to 16 (the row's q and dout are staged once per workgroup), fewer
    // when that leaves under about one workgroup per CU
    const int nb = (a.n_idx + 31) / 32;
    const int bpw = (int)std::min<int64_t>(kDkvBpwMax, std::max<int64_t>(2, ((int64_t)nb * T + 255) / 256));
    const dim3 grid((nb + bpw - 1) / bpw, T);
    if (hk == 4) launch_kernel(k_sparse_mla_bwd_dkv_rows<DQK, 4>, grid, dim3(512), st, a, bpw);
    else launch_kernel(k_sparse_mla_bwd_dkv_rows<DQK, 8>, grid, dim3(512), st, a, bpw);
    return;
  }
  const int cg = hk >= 16 ? 2 : 3;
  const dim3 grid((CT + cg - 1) / cg, T);
  if (hk == 4) launch_kernel(k_sparse_mla_bwd_dkv<DQK, 4>, grid, dim3(256), st, a, cg);
  else if (hk == 8) launch_kernel(k_sparse_mla_bwd_dkv<DQK, 8>, grid, dim3(256), st, a, cg);
  else launch_kernel(k_sparse_mla_bwd_dkv<DQK, 16>, grid, dim3(256), st, a, cg);
}

hipError_t launch_sparse_mla_bwd(const MlaBwdArgs& a, int d_qk, int T, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  const bool fused = a.Hp == 16;
  // 16-head groups: one workgroup (4 waves) when fused, else two groups per workgroup (8 waves)
  const dim3 grid(fused ? 1 : a.Hp / 32, T, fused ? 1 : a.nsplit);
  const dim3 block(fused ? 256 : 512);
  if (d_qk == 576) {
    if (fused) launch_kernel(k_sparse_mla_bwd<576, true>, grid, block, st, a);
    else launch_kernel(k_sparse_mla_bwd<576, false>, grid, block, st, a);
  } else {
    if (fused) launch_kernel(k_sparse_mla_bwd<512, true>, grid, block, st, a);
    else launch_kernel(k_sparse_mla_bwd<512, false>, grid, block, st, a);
  }
  return hipGetLastError();
}

int bwd_splits(int T, int Hp, int n_idx) {
  if (Hp <= 16 || T <= 0) return 1;
  const int64_t wgs = (int64_t)T * (Hp / 32);
  int n = (int)std::min<int64_t>(4, (256 + wgs - 1) / wgs);
  return std::max(1, std::min(n, n_idx / 256));
}

hipError_t launch_sparse_mla_bwd_mid(const MlaBwdArgs& a, int d_qk, int T, hipStream_t st) {
  if (T <= 0 || a.Hp == 16) return hipSuccess;
  const int nbm = a.ws_owner && a.n_idx > 0 ? (int)(((int64_t)T * a.n_idx + 255) / 256) : 0;
  const int nbd = a.nsplit > 1 ? (int)(((int64_t)T * a.H * d_qk / 4 + 255) / 256) : 0;
  if (nbm + nbd == 0) return hipSuccess;
  launch_kernel(k_sparse_mla_bwd_mid, dim3(nbm + nbd), dim3(256), st, a, T, d_qk, nbm);
  return hipGetLastError();
}

hipError_t launch_sparse_mla_bwd_dkv(const MlaBwdArgs& a, int d_qk, int T, hipStream_t st) {
  if (T <= 0 || a.n_idx <= 0 || a.Hp == 16) return hipSuccess;   // 16 heads: fused above
  if (d_qk == 576) launch_dkv<576>(a, T, st);
  else launch_dkv<512>(a, T, st);
  return hipGetLastError();
}

}  // namespace dsa
