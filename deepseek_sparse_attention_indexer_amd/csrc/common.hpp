// Device helpers shared by the DSA kernels (gfx950 / CDNA4 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;

namespace dsa {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// 16x16x32 bf16 MFMA. Lane l supplies A[l%16][8(l/16)+j] and B[8(l/16)+j][l%16] (j = 0..7)
// and receives C[4(l/16)+r][l%16] (r = 0..3); verified on gfx950 by an in-bounds probe.
__device__ __forceinline__ f32x4_t mfma_bf16_16x16x32(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// 32x32x16 bf16 MFMA. Lane l supplies A[l%32][8(l/32)+j] and B[8(l/32)+j][l%32] (j = 0..7)
// and receives C[8(r/4) + 4(l/32) + r%4][l%32] in accumulator r = 0..15; verified on gfx950 by
// an in-bounds probe against a host product.
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
__device__ __forceinline__ f32x16_t mfma_bf16_32x32x16(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Reduce-scatter of four per-lane partials over the four 16-lane rows of a wave: p_j at lane
// 16 g + c holds row g's share of item 16 j + c, and lane l receives the sum over g of p_{l/16}
// at lane 16 g + l % 16. gfx950's lane swaps do the exchange in the vector ALU (permlane32_swap:
// lanes 32..63 of the first operand trade places with lanes 0..31 of the second; permlane16_swap:
// the odd 16-lane rows of the first with the even rows of the second); each add then sums the
// same two values an xor-32 / xor-16 lane exchange would.
__device__ __forceinline__ float reduce_scatter_rows4(float p0, float p1, float p2, float p3) {
  const auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(p0), __float_as_uint(p2), false, false);
  const auto y = __builtin_amdgcn_permlane32_swap(__float_as_uint(p1), __float_as_uint(p3), false, false);
  const float k0 = __uint_as_float(x[0]) + __uint_as_float(x[1]);
  const float k1 = __uint_as_float(y[0]) + __uint_as_float(y[1]);
  const auto z = __builtin_amdgcn_permlane16_swap(__float_as_uint(k0), __float_as_uint(k1), false, false);
  return __uint_as_float(z[0]) + __uint_as_float(z[1]);
}

// max of x and its lane-xor-32 / lane-xor-16 partner, by the lane swaps (no LDS round trip)
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Paging of a token cache, resolved on the host into device-friendly fields.
struct Paging {
  const int32_t* bt;      // block table or nullptr
  const int32_t* req_base;
  int64_t bt_stride;
  int64_t n_slots;        // tokens in the cache (pages * page_size when paged)
  int32_t page;           // tokens per page
  int32_t page_shift;     // log2(page) if a power of two, else -1
  int32_t n_pages;        // n_slots / page
  int32_t _pad;
};

// Logical position s of request b -> slot, clamped into the cache (a table entry or a
// position outside the caller's contract yields some in-cache slot, never a wild address).
__device__ __forceinline__ int64_t slot_of(const Paging& p, int b, int s) {
  if (p.bt) {
    int lp, off;
    if (p.page_shift >= 0) { lp = s >> p.page_shift; off = s & (p.page - 1); }
    else { lp = s / p.page; off = s - lp * p.page; }
    lp = min(max(lp, 0), (int)p.bt_stride - 1);
    int pg = p.bt[(int64_t)b * p.bt_stride + lp];
    pg = min(max(pg, 0), p.n_pages - 1);
    return (int64_t)pg * p.page + off;
  }
  int64_t sl = (int64_t)p.req_base[b] + s;
  return sl < 0 ? 0 : (sl >= p.n_slots ? p.n_slots - 1 : sl);
}

// Bf16 rows in LDS. gfx950's LDS has 128 four-byte banks (512 bytes); a 16-byte read is served
// 32 lanes at a time and an 8-byte transposing read all 64 lanes at once (both measured with
// the LDS bank-conflict counter). Rows laid at a stride of 64 (mod 128) bytes put 8
// consecutive rows, and rows 4 apart, in distinct 64-byte bank groups; with 16-byte chunk q of
// row r stored at chunk q ^ row_swz(r), rows r and r + 8 also take different banks for a read
// of 16 rows at one 16-byte column (the score product's A operand).
__device__ __forceinline__ int row_swz(int r) { return (r >> 2) & 2; }

// Workgroup barrier for LDS traffic only: waits for this wave's LDS operations, then the
// barrier. __syncthreads() also waits for every outstanding global load of the wave (vmcnt 0),
// which would turn a prefetch issued before the barrier into a stall. Not for data written to
// LDS by direct global->LDS loads (those complete on vmcnt).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// s_waitcnt vmcnt(N) alone (expcnt and lgkmcnt fields at their maxima: not waited on)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
// the same for a wave-uniform count in [LO, HI], by a binary search of scalar branches
template <int LO, int HI>
__device__ __forceinline__ void wait_vmcnt_dyn(int n) {
  if constexpr (LO == HI) {
    wait_vmcnt<LO>();
  } else {
    constexpr int MID = (LO + HI) / 2;
    if (n <= MID) wait_vmcnt_dyn<LO, MID>(n);
    else wait_vmcnt_dyn<MID + 1, HI>(n);
  }
}

// One of two pagings, field by field (selecting a reference would put both in scratch).
__device__ __forceinline__ Paging pick_paging(bool x, const Paging& p1, const Paging& p0) {
  Paging r;
  r.bt = x ? p1.bt : p0.bt;
  r.req_base = x ? p1.req_base : p0.req_base;
  r.bt_stride = x ? p1.bt_stride : p0.bt_stride;
  r.n_slots = x ? p1.n_slots : p0.n_slots;
  r.page = x ? p1.page : p0.page;
  r.page_shift = x ? p1.page_shift : p0.page_shift;
  r.n_pages = x ? p1.n_pages : p0.n_pages;
  r._pad = 0;
  return r;
}

// The same mapping in two steps, so that many table reads are in flight before any is used
// and no branch separates a read from its use (a merge after a conditional read makes the
// compiler wait right there): slot_read issues the block-table read (a packed cache reads
// req_base[b] through the same load), slot_done clamps into the cache. s >= 0.
struct SlotRead {
  int ent;
  int off;
};
__device__ __forceinline__ SlotRead slot_read(const Paging& p, int b, int s) {
  const bool paged = p.bt != nullptr;
  const int q = p.page_shift >= 0 ? (s >> p.page_shift) : s / p.page;
  const int lp = min(max(q, 0), max((int)p.bt_stride - 1, 0));
  SlotRead r;
  r.off = paged ? s - q * p.page : s;
  const int32_t* tb = paged ? p.bt : p.req_base;
  r.ent = tb[paged ? (int64_t)b * p.bt_stride + lp : (int64_t)b];
  return r;
}
__device__ __forceinline__ int64_t slot_done(const Paging& p, SlotRead r) {
  const int64_t in_page = (int64_t)min(max(r.ent, 0), p.n_pages - 1) * p.page + r.off;
  const int64_t v = (int64_t)r.ent + r.off;
  const int64_t packed = v < 0 ? 0 : (v >= p.n_slots ? p.n_slots - 1 : v);
  return p.bt != nullptr ? in_page : packed;
}

// max(0, x) for any fp32 x in one integer max: a float with the sign bit clear is a
// non-negative int32 and keeps its bits; every negative float (and -0) is a negative int32 and
// becomes +0. fmaxf would first canonicalise an MFMA result (a second instruction).
__device__ __forceinline__ float relu_f32(float x) {
  return __int_as_float(max(__float_as_int(x), 0));
}

// Order-preserving map fp32 -> uint32 (larger float -> larger key); -0 and +0 share a key.
__device__ __forceinline__ uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (f == 0.0f) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Two fp32 that are exactly representable in bf16 -> packed bf16 pair (lo in bits 0..15).
__device__ __forceinline__ uint32_t pack_bf16_exact(float lo, float hi) {
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// Two fp32 -> packed bf16 pair (lo in bits 0..15), round-to-nearest-even: one gfx950
// v_cvt_pk_bf16_f32 (checked on the GPU bit for bit against the integer rounding
// (u + 0x7fff + ((u >> 16) & 1)) >> 16 over 2^25 finite patterns, denormals and ties included).
// Transposing LDS read of 16-bit data (gfx950 ds_read_b64_tr_b16). Each lane addresses a piece
// of four consecutive elements (8-byte aligned); in each group of 16 lanes, lane 4 a + b
// receives element b of the pieces of lanes a, a + 4, a + 8 and a + 12 of its group, in that
// order (lane layout measured on the hardware).
__device__ __forceinline__ u32x2_t ds_read_tr16(const uint16_t* p) {
  typedef short s16x4_t __attribute__((ext_vector_type(4)));
  auto* lp = reinterpret_cast<__attribute__((address_space(3))) s16x4_t*>(reinterpret_cast<uintptr_t>(p) & 0xffffffffu);
  return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(lp));
}

__device__ __forceinline__ uint32_t pack_bf16_rne(float lo, float hi) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

__device__ __forceinline__ uint32_t bf16_rne_bits(float f) { return pack_bf16_rne(f, 0.f) & 0xFFFFu; }

// 2^x by the hardware exponential (v_exp_f32). exp2f adds a rescaling around it only so that
// results below 2^-126 come out as exact denormals; softmax weights that small vanish against
// a sum whose largest term is at least 2^-8, so the hot loops take the bare instruction.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// 4 OCP e4m3 bytes -> 4 floats (gfx950's conversion is the OCP e4m3fn decode).
__device__ __forceinline__ void fp8x4_to_f32(uint32_t w, float* o) {
  f32x2_t a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  f32x2_t b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  o[0] = a[0]; o[1] = a[1]; o[2] = b[0]; o[3] = b[1];
}

// 8 fp8 bytes -> 8 bf16 (exact: an e4m3 value has 4 significant bits and fits bf16's range).
__device__ __forceinline__ u32x4_t fp8x8_to_bf16x8(u32x2_t raw) {
  float f[8];
  fp8x4_to_f32(raw[0], f);
  fp8x4_to_f32(raw[1], f + 4);
  u32x4_t r;
  r[0] = pack_bf16_exact(f[0], f[1]);
  r[1] = pack_bf16_exact(f[2], f[3]);
  r[2] = pack_bf16_exact(f[4], f[5]);
  r[3] = pack_bf16_exact(f[6], f[7]);
  return r;
}

// 4 fnuz e4m3 bytes (exponent bias 8, largest magnitude 240) -> fp32, exactly. Moving a
// byte's sign to bit 31 and its exponent and mantissa fields to bits 30..20 gives an fp32 whose
// value is the byte's times 2^-119 (subnormal codes land on fp32 denormals, which the build
// preserves); the product with 2^119 is then exact. There is no native conversion of this
// encoding on gfx950. Byte 0x80 (NaN in this encoding) decodes as -0.
__device__ __forceinline__ void fnuz4_to_f32(uint32_t w, float* o) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t b = (w >> (8 * i)) & 0xffu;
    o[i] = __uint_as_float(((b & 0x80u) << 24) | ((b & 0x7fu) << 20)) * 0x1p119f;
  }
}

// 2^(e-127) for a UE8M0 byte 1..254 (exact, built from the exponent field).
__device__ __forceinline__ float ue8m0_scale(uint32_t e) { return __uint_as_float(e << 23); }

// Two OCP e4m3 bytes (bytes 0-1 of w, or 2-3 with HI) -> two bf16 (low half = the lower byte)
// times 2^(exponent field of s): gfx950's scaled conversion applies only the exponent of its
// fp32 scale, so for a power-of-two scale the result is the exact product.
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2_pow2(uint32_t w, float s) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, s, HI));
}

template <typename T>
__device__ __forceinline__ T wave_bcast_first(T v) {
  return __builtin_amdgcn_readfirstlane(v);
}

}  // namespace dsa
