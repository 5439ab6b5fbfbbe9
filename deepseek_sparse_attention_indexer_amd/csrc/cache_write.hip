// Cache writes on gfx950: bf16 rows -> the formats the layer reads.
//
// Formats of aiter PR 4382 "Paged Sparse Attention Gluon Kernel" (section "Supported formats
// & dtypes"): the uniform fp8 pool (e4m3 values, one fp32 scale per 64 channels; OCP or, per
// the section "fp8 flavors", fnuz bytes: bias 8, largest magnitude 240), the packed
// fp8_ds_mla token (448 NoPE channels as e4m3 with one UE8M0 exponent per 64 channels, 64 RoPE
// channels as bf16; page-planar, 584 bytes per token), and fp8 index keys with one fp32 scale
// per token; plus plain bf16 copies. Rounding (the pages state the layouts only):
//   * e4m3: round to nearest even after saturating to +-448 (gfx950's conversion); fnuz
//     likewise after saturating to +-240, and zero is always 0x00 (0x80 is NaN there);
//   * fp32 scales: amax / 448 (fnuz: amax / 240) in fp32 (1 for an all-zero group), values
//     divided by the scale with IEEE round-to-nearest division;
//   * UE8M0: the smallest k with 448 * 2^k >= amax, found exactly from amax's exponent and
//     mantissa bits, stored as k + 127 in [1, 254] (127 for an all-zero group); the division
//     by 2^k is an exact ldexp.
//
// One wave per token; lane l holds channels [8 l, 8 l + 8) of each 512-channel pass (one
// 16-byte load), so a 64-channel group is 8 consecutive lanes and its maximum takes three
// lane exchanges. A slot outside [0, n_slots) (or -1) is skipped: nothing is written for it.
#include "common.hpp"
#include "kernels.hpp"

namespace dsa {

constexpr int kCwWaves = 4;   // tokens per workgroup

__device__ __forceinline__ float lanes_max(float v, int lanes) {
  for (int d = 1; d < lanes; d <<= 1) v = fmaxf(v, __shfl_xor(v, d));
  return v;
}

__device__ __forceinline__ void bf16x8_to_f32(u32x4_t v, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(v[i] << 16);
    f[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
  }
}

// 8 floats (already within +-448) -> 8 e4m3 bytes, value i in byte i
__device__ __forceinline__ u32x2_t f32x8_to_fp8(const float* f) {
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], lo, true);
  int hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[4], f[5], 0, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[6], f[7], hi, true);
  return u32x2_t{(uint32_t)lo, (uint32_t)hi};
}

__device__ __forceinline__ float sat448(float x) { return fminf(fmaxf(x, -448.0f), 448.0f); }

// 8 floats (already within +-240) -> 8 fnuz e4m3 bytes. A fnuz code's value is half that of
// the OCP code with the same bits, on the same grid, so the OCP conversion of 2y gives the
// fnuz byte of y except at the two ends: |y| in (232, 240] rounds to 240 (code 0x7F, NaN in
// OCP): the conversion of the saturated 2y gives 0x7E and bit 0 is set; and values that round
// to zero convert as +0 (OCP's -0 byte is fnuz's NaN).
__device__ __forceinline__ u32x2_t f32x8_to_fnuz(const float* y) {
  float f2[8];
  uint32_t big[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float a = fabsf(y[i]);
    float v = sat448(2.f * y[i]);
    v = a <= 0x1p-11f ? 0.f : v;                 // |2y| <= 2^-10 rounds to zero
    f2[i] = v;
    if (a > 232.f) big[i >> 2] |= 1u << (8 * (i & 3));
  }
  u32x2_t r = f32x8_to_fp8(f2);
  r[0] |= big[0];
  r[1] |= big[1];
  return r;
}

template <int KIND>
__global__ __launch_bounds__(64 * kCwWaves) void k_cache_write(CacheWriteArgs a) {
  const int lane = threadIdx.x & 63;
  const int tok = blockIdx.x * kCwWaves + (threadIdx.x >> 6);
  if (tok >= a.n_tok) return;                               // whole wave
  const int64_t slot = a.slots[tok];
  if (slot < 0 || slot >= a.n_slots) return;                // whole wave: skipped
  const uint16_t* src = a.src + (int64_t)tok * a.ld_src;

  if constexpr (KIND == kCwBf16) {
    // plain copy of D bf16 channels, 16 bytes per lane and step
    uint16_t* dst = reinterpret_cast<uint16_t*>(a.data) + slot * a.D;
    for (int c = 8 * lane; c < a.D; c += 512)
      *reinterpret_cast<u32x4_t*>(dst + c) = *reinterpret_cast<const u32x4_t*>(src + c);
  } else if constexpr (KIND == kCwScaled || KIND == kCwScaledFnuz) {
    // e4m3 with one fp32 scale per `group` channels (uniform pool: 64; index keys: the row)
    constexpr float kMax = KIND == kCwScaled ? 448.0f : 240.0f;
    const int lanes = a.group / 8;                          // lanes per group (8 or 16)
    uint8_t* dst = a.data + slot * a.D;
    for (int c0 = 0; c0 < a.D; c0 += 512) {                 // uniform over the wave
      const int c = c0 + 8 * lane;
      const bool live = c < a.D;
      float f[8];
      if (live) {
        bf16x8_to_f32(*reinterpret_cast<const u32x4_t*>(src + c), f);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = 0.f;
      }
      float m = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(f[i]));
      m = lanes_max(m, lanes);
      const float scale = m > 0.f ? __fdiv_rn(m, kMax) : 1.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) f[i] = fminf(fmaxf(__fdiv_rn(f[i], scale), -kMax), kMax);
      if (live) {
        *reinterpret_cast<u32x2_t*>(dst + c) = KIND == kCwScaled ? f32x8_to_fp8(f) : f32x8_to_fnuz(f);
        if ((c % a.group) == 0) a.fscale[slot * (a.D / a.group) + c / a.group] = scale;
      }
    }
  } else {  // kCwDsMla: 448 NoPE channels (lanes 0..55) + 64 RoPE bf16 channels (lanes 56..63)
    const int P = a.page;
    const int64_t page = slot / P;
    const int64_t pos = slot - page * P;
    uint8_t* pbase = a.data + page * (int64_t)P * 584;
    uint8_t* dtok = pbase + pos * 576;
    uint8_t* etok = pbase + (int64_t)P * 576 + pos * 8;
    const u32x4_t raw = *reinterpret_cast<const u32x4_t*>(src + 8 * lane);
    float f[8];
    bf16x8_to_f32(raw, f);
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(f[i]));
    m = lanes_max(m, 8);
    // smallest k with 448 * 2^k >= m: m = 1.f * 2^E, 448 = 1.75 * 2^8, so k = E - 8 when
    // 1.f <= 1.75, else E - 7; subnormal maxima clamp to the smallest exponent byte
    int ebyte = 127;
    if (m > 0.f) {
      const uint32_t u = __float_as_uint(m);
      const int ef = (int)(u >> 23);
      int k = -300;
      if (ef != 0) k = (u & 0x7fffffu) <= 0x600000u ? (ef - 127) - 8 : (ef - 127) - 7;
      ebyte = min(max(k + 127, 1), 254);
    }
    if (lane < 56) {
#pragma unroll
      for (int i = 0; i < 8; ++i) f[i] = sat448(__builtin_amdgcn_ldexpf(f[i], 127 - ebyte));
      *reinterpret_cast<u32x2_t*>(dtok + 8 * lane) = f32x8_to_fp8(f);
      if ((lane & 7) == 0) etok[lane >> 3] = (uint8_t)ebyte;
    } else {
      // RoPE bf16 bytes after the 448 NoPE bytes (8-byte stores: the page base is only
      // 8-byte aligned for odd page sizes)
      uint8_t* d = dtok + 448 + 16 * (lane - 56);
      *reinterpret_cast<u32x2_t*>(d) = u32x2_t{raw[0], raw[1]};
      *reinterpret_cast<u32x2_t*>(d + 8) = u32x2_t{raw[2], raw[3]};
      if (lane == 56) etok[7] = 0;
    }
  }
}

hipError_t launch_cache_write(const CacheWriteArgs& a, int kind, hipStream_t st) {
  if (a.n_tok <= 0) return hipSuccess;
  const dim3 grid((a.n_tok + kCwWaves - 1) / kCwWaves);
  if (kind == kCwBf16) launch_kernel(k_cache_write<kCwBf16>, grid, dim3(64 * kCwWaves), st, a);
  else if (kind == kCwScaled) launch_kernel(k_cache_write<kCwScaled>, grid, dim3(64 * kCwWaves), st, a);
  else if (kind == kCwScaledFnuz) launch_kernel(k_cache_write<kCwScaledFnuz>, grid, dim3(64 * kCwWaves), st, a);
  else launch_kernel(k_cache_write<kCwDsMla>, grid, dim3(64 * kCwWaves), st, a);
  return hipGetLastError();
}

}  // namespace dsa
