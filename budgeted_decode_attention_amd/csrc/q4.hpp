// 4-bit cache slots (gfx950 device helpers).
//
// Scissorhands summary page, Abstract: the budgeted cache combines with 4-bit
// quantisation.  The page fixes no format; the one used here: a row of d
// elements is d / 32 groups of 32 consecutive elements, each with a float32
// scale = (largest magnitude) * fl32(1/7) and codes c = rint(x / scale) in
// [-7, 7] (float32 quotient, correctly rounded, then rounded half to even; a
// zero scale gives codes 0).  A slot row reads back as c * scale.
//
// Storage: the d / 2 code bytes of a row hold element 2b of byte b in the low
// nibble and element 2b + 1 in the high nibble, each as c + 8 (1..15); the
// scales of a row are d / 32 consecutive floats.  A group's codes are 16
// bytes.  The prefill gather quantises one group per lane (one 16-byte store,
// many rows in parallel); the decode step's single new row is quantised with
// one element per lane; the decode kernels read half a group per lane.
#pragma once

#include "common.hpp"

namespace kve {

constexpr int kQGroup = 32;
constexpr float kInvQMax = (float)(1.0 / 7.0);

// n consecutive elements of the storage dtype at p (16-byte aligned) as floats.
template <int DT, int N>
__device__ inline void load_elems(const void* p, float* f) {
  constexpr int EPL = St<DT>::EPL;
  static_assert(N % EPL == 0, "whole 16-byte loads");
#pragma unroll
  for (int i = 0; i < N / EPL; ++i) St<DT>::unpack(ld16((const char*)p + i * 16), f + i * EPL);
}

// One group x[0, 32) -> its 16 code bytes and its scale.  Every decision is a
// float32 operation with one rounding: the product for the scale, the
// quotient (__fdiv_rn), the round to nearest even (rintf).
__device__ inline void q4_quantize(const float* x, uint4& packed, float& scale) {
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < kQGroup; ++j) amax = fmaxf(amax, fabsf(x[j]));
  scale = __fmul_rn(amax, kInvQMax);
  uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int j = 0; j < kQGroup; ++j) {
    float c = scale > 0.f ? rintf(__fdiv_rn(x[j], scale)) : 0.f;
    c = fminf(fmaxf(c, -7.f), 7.f);
    w[j >> 3] |= (uint32_t)((int)c + 8) << ((j & 7) * 4);
  }
  packed = make_uint4(w[0], w[1], w[2], w[3]);
}

// The eight stored nibbles (c + 8) of one little-endian code word, in element
// order, as floats.  Masking every other nibble into byte lanes lets
// each element convert with one unsigned-byte-to-float conversion.  The
// empty asm statements hide the masks from the optimizer, which would
// otherwise fold them into one bit-field extract per nibble (two vector
// instructions per element instead of one).
__device__ inline void q4_nibbles(uint32_t w, float* f) {
  uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
  asm("" : "+v"(lo));
  asm("" : "+v"(hi));
  f[0] = (float)(lo & 0xffu);
  f[1] = (float)(hi & 0xffu);
  f[2] = (float)((lo >> 8) & 0xffu);
  f[3] = (float)((hi >> 8) & 0xffu);
  f[4] = (float)((lo >> 16) & 0xffu);
  f[5] = (float)((hi >> 16) & 0xffu);
  f[6] = (float)(lo >> 24);
  f[7] = (float)(hi >> 24);
}

// The same quantisation with one element per lane: lanes e of a row (e in
// [0, D), 32 consecutive lanes per group, whole waves) each hold x = element
// e; the group's largest magnitude comes from a butterfly over its 32 lanes,
// the code from the lane's own quotient, and eight lanes' nibbles are merged
// into one 32-bit word, stored by the group's lanes with e % 8 == 0.
__device__ inline void q4_quantize_lane(float x, int e, char* dst, float* dsc) {
  float amax = fabsf(x);
#pragma unroll
  for (int o = 16; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  const float scale = __fmul_rn(amax, kInvQMax);
  float c = scale > 0.f ? rintf(__fdiv_rn(x, scale)) : 0.f;
  c = fminf(fmaxf(c, -7.f), 7.f);
  uint32_t w = (uint32_t)((int)c + 8) << ((e & 7) * 4);
#pragma unroll
  for (int o = 1; o < 8; o <<= 1) w |= (uint32_t)__shfl_xor((int)w, o);
  if ((e & 7) == 0) reinterpret_cast<uint32_t*>(dst)[e >> 3] = w;
  if ((e & (kQGroup - 1)) == 0) dsc[e / kQGroup] = scale;
}

// Quantises the row of D elements at src (storage dtype) into code bytes dst
// and scales dsc, group g = the calling lane's `g`.
template <int DT, int D>
__device__ inline void q4_store_group(const void* src, char* dst, float* dsc, int g) {
  float x[kQGroup];
  load_elems<DT, kQGroup>((const char*)src + (size_t)g * kQGroup * (16 / St<DT>::EPL), x);
  uint4 pk;
  float sc;
  q4_quantize(x, pk, sc);
  st16(dst + g * 16, pk);
  dsc[g] = sc;
}

}  // namespace kve
