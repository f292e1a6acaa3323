// Device helpers shared by the kvevict kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.hpp"

namespace kve {

constexpr int kWave = 64;

// ---------------------------------------------------------------- storage types
// A 16-byte load carries EPL elements of the storage dtype.
template <int DT> struct St;

template <> struct St<F32> {
  static constexpr int EPL = 4;
  __device__ static inline void unpack(const uint4& r, float* f) {
    f[0] = __uint_as_float(r.x); f[1] = __uint_as_float(r.y);
    f[2] = __uint_as_float(r.z); f[3] = __uint_as_float(r.w);
  }
};

template <> struct St<BF16> {
  static constexpr int EPL = 8;
  __device__ static inline void unpack(const uint4& r, float* f) {
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};

template <> struct St<F16> {
  static constexpr int EPL = 8;
  __device__ static inline void unpack(const uint4& r, float* f) {
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      _Float16 lo = __builtin_bit_cast(_Float16, (uint16_t)(w[i] & 0xffffu));
      _Float16 hi = __builtin_bit_cast(_Float16, (uint16_t)(w[i] >> 16));
      f[2 * i] = (float)lo;
      f[2 * i + 1] = (float)hi;
    }
  }
};

template <int DT> constexpr int elem_bytes() { return 16 / St<DT>::EPL; }

// Element i of a storage-dtype row as a float.
template <int DT>
__device__ inline float load_elem(const void* row, int i) {
  if constexpr (DT == F32) {
    return reinterpret_cast<const float*>(row)[i];
  } else if constexpr (DT == BF16) {
    return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(row)[i] << 16);
  } else {
    return (float)__builtin_bit_cast(_Float16, reinterpret_cast<const uint16_t*>(row)[i]);
  }
}

__device__ inline uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ inline void st16(void* p, const uint4& v) { *reinterpret_cast<uint4*>(p) = v; }

// ---------------------------------------------------------------- lane-group sums
// Sum over aligned groups of G lanes (G in {2, 4, 8, 16, 32}); every lane of the
// group receives the group's sum.  Within a 16-lane row the partners come from
// DPP permutations (quad swaps, then the half-row and row mirrors), which pair
// each lane with one holding the other half of the partial sums at each step.
template <int CTRL> __device__ inline float dpp_add(float v) {
  return v + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}

template <int G> __device__ inline float group_sum(float v) {
  static_assert(G == 2 || G == 4 || G == 8 || G == 16 || G == 32, "group size");
  v = dpp_add<0xB1>(v);        // quad_perm [1,0,3,2]
  if constexpr (G >= 4) v = dpp_add<0x4E>(v);    // quad_perm [2,3,0,1]
  if constexpr (G >= 8) v = dpp_add<0x141>(v);   // row_half_mirror
  if constexpr (G >= 16) v = dpp_add<0x140>(v);  // row_mirror
  if constexpr (G >= 32) v += __shfl_xor(v, 16);
  return v;
}

// ---------------------------------------------------------------- wave / block reductions
__device__ inline float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ inline double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Result broadcast to every thread.  `scratch` needs NT / 64 entries and is
// reused after a barrier.
template <int NT> __device__ inline float block_max(float v, float* scratch) {
  v = wave_max(v);
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) scratch[w] = v;
  __syncthreads();
  float r = scratch[0];
#pragma unroll
  for (int i = 1; i < NT / kWave; ++i) r = fmaxf(r, scratch[i]);
  __syncthreads();
  return r;
}

template <int NT> __device__ inline double block_sum(double v, double* scratch) {
  v = wave_sum(v);
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) scratch[w] = v;
  __syncthreads();
  double r = scratch[0];
#pragma unroll
  for (int i = 1; i < NT / kWave; ++i) r += scratch[i];
  __syncthreads();
  return r;
}

// Lexicographic minimum of (score, position); ties in both keep the smaller
// slot.  Empty candidates carry score +inf.
struct MinKey {
  double s;
  int32_t pos;
  int32_t slot;
};

__device__ inline bool key_less(const MinKey& a, const MinKey& b) {
  if (a.s != b.s) return a.s < b.s;
  if (a.pos != b.pos) return a.pos < b.pos;
  return a.slot < b.slot;
}

__device__ inline MinKey wave_argmin(MinKey k) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    MinKey other;
    other.s = __shfl_xor(k.s, o);
    other.pos = __shfl_xor(k.pos, o);
    other.slot = __shfl_xor(k.slot, o);
    if (key_less(other, k)) k = other;
  }
  return k;
}

template <int NT> __device__ inline MinKey block_argmin(MinKey k, MinKey* scratch) {
  k = wave_argmin(k);
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) scratch[w] = k;
  __syncthreads();
  MinKey r = scratch[0];
#pragma unroll
  for (int i = 1; i < NT / kWave; ++i)
    if (key_less(scratch[i], r)) r = scratch[i];
  __syncthreads();
  return r;
}

__device__ inline bool token_kept(const uint32_t* bitmap, int vocab, int id) {
  if (id < 0 || id >= vocab || bitmap == nullptr) return false;
  return (bitmap[id >> 5] >> (id & 31)) & 1u;
}

// Whether token `id` is protected under id mode `mode`.
__device__ inline bool id_protected(int mode, const IdSets& s, int id) {
  switch (mode) {
    case IDS_SPECIAL: return token_kept(s.special, s.vocab, id);
    case IDS_SPECIAL_PUNCT: return token_kept(s.special, s.vocab, id) || token_kept(s.punct, s.vocab, id);
    case IDS_KEEP: return token_kept(s.keep, s.vocab, id);
  }
  return false;
}

}  // namespace kve
