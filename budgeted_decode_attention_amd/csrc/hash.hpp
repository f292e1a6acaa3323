// HashEvict helpers shared by the replacement kernels and the fused decode
// (HashEvict summary page, original abstract: sign sketches of a Gaussian
// projection, Hamming distance to the query's sketch, the farthest key
// replaced before attention).  Workgroups of kHashNT threads.
#pragma once

#include "common.hpp"
#include "q4.hpp"

namespace kve {

constexpr int kHashNT = 256;

template <int BITS> struct SkWord { using T = uint32_t; };
template <> struct SkWord<64> { using T = uint64_t; };
__device__ inline int popcnt(uint32_t x) { return __popc(x); }
__device__ inline int popcnt(uint64_t x) { return __popcll(x); }

// The BITS-bit field of a wave ballot that starts at lane `first`.
template <int BITS> __device__ inline typename SkWord<BITS>::T ballot_field(uint64_t m, int first) {
  if constexpr (BITS == 64) return m;
  else return (typename SkWord<BITS>::T)((m >> first) & ((1ull << BITS) - 1ull));
}

__device__ inline double bf16_to_double(uint16_t w) { return (double)__uint_as_float((uint32_t)w << 16); }

// Exact sign of sum_i a_i b_i (each product exact in float64), by growing a
// zero-free non-overlapping expansion with two-sum; e holds up to D + 1
// components (LDS, owned by the calling lane while it runs).  Rarely taken.
template <int DT, int D>
__device__ inline int exact_sign(const char* row, const uint16_t* W, int bits, int b, double* e) {
  int len = 0;
  for (int i = 0; i < D; ++i) {
    double q = (double)load_elem<DT>(row, i) * bf16_to_double(W[i * bits + b]);
    int k = 0;
    for (int j = 0; j < len; ++j) {
      const double s = q + e[j];
      const double bv = s - q;
      const double av = s - bv;
      const double err = (q - av) + (e[j] - bv);
      q = s;
      if (err != 0.0) e[k++] = err;
    }
    if (q != 0.0) e[k++] = q;
    len = k;
  }
  if (len == 0) return 0;
  return e[len - 1] > 0.0 ? 1 : 0;   // the largest component carries the sign
}

// Bytes of LDS one wave needs for the exact fallback.
template <int D> __host__ __device__ constexpr size_t exact_lds() { return (size_t)(D + 1) * 8; }

// Sign bit b of a row: float64 dot with the error bound; -1 if the bound does
// not settle the sign.  xs(i): element i of the row as a float (from LDS or
// global memory), Ws: the projection as bf16 bits.
template <int D, typename X>
__device__ inline int sketch_bit_fast(X xs, const uint16_t* Ws, int bits, int b) {
  double s = 0.0, a = 0.0;
#pragma unroll 8
  for (int i = 0; i < D; ++i) {
    const double x = (double)xs(i);
    const double w = bf16_to_double(Ws[i * bits + b]);
    s = fma(x, w, s);
    a = fma(fabs(x), fabs(w), a);
  }
  // |s - exact| <= gamma_D * sum|terms|; sum|terms| itself is computed with a
  // relative error below gamma_D, so gamma_{2D+2} bounds the comparison.
  constexpr double u = 1.1102230246251565e-16;
  constexpr double g = (2 * D + 2) * u / (1.0 - (2 * D + 2) * u);
  if (fabs(s) > g * a) return s > 0.0 ? 1 : 0;
  return -1;
}

// Sign bit b of `row` (the exact sign of sum_i W[i][b] row[i]), called by
// every lane of a wave (lanes with active == false take no part but must
// call).  The float64 bound settles almost every bit; the lanes it does not
// settle re-add their terms exactly, one lane at a time, in the wave's LDS
// buffer ebuf (exact_lds<D>() bytes) -- so no lane needs private memory.
// The exact path re-reads the row and projection from global memory.
template <int DT, int D>
__device__ inline int sketch_bit(bool active, const float* xs, const uint16_t* Ws, const char* row,
                                 const uint16_t* W, int bits, int b, double* ebuf) {
  int bit = active ? sketch_bit_fast<D>([&](int i) { return xs[i]; }, Ws, bits, b) : 0;
  uint64_t fr = __ballot(bit < 0);
  const int lane = threadIdx.x & (kWave - 1);
  while (fr) {                                   // uniform over the wave
    const int L = __builtin_ctzll(fr);
    if (lane == L) bit = exact_sign<DT, D>(row, W, bits, b, ebuf);
    fr &= fr - 1;
  }
  return bit;
}

// Copies the [D][BITS] bf16 projection into LDS (all threads of the workgroup).
template <int D, int BITS>
__device__ inline void stage_proj(uint16_t* Ws, const uint16_t* W) {
  for (int i = threadIdx.x; i < D * BITS / 8; i += kHashNT)
    reinterpret_cast<uint4*>(Ws)[i] = reinterpret_cast<const uint4*>(W)[i];
}

// Eviction keys: distance << 16 | (65535 - position).  The maximum is the
// farthest key, then the oldest position; positions in a cache are distinct
// and below 65536, so a non-zero maximum is unique.  Lanes without a
// candidate hold 0.
__device__ inline uint32_t evict_key(uint32_t dist, int pos) { return (dist << 16) | (uint32_t)(0xFFFF - pos); }
__device__ inline int key_position(uint32_t key) { return 0xFFFF - (int)(key & 0xFFFF); }

// The wave's largest key (every lane receives it): DPP within each 16-lane
// row, then the four rows' values.
__device__ inline uint32_t wave_max_key(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false));    // quad_perm [1,0,3,2]
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false));    // quad_perm [2,3,0,1]
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false));   // row_half_mirror
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, false));   // row_mirror
  return max(max((uint32_t)__builtin_amdgcn_readlane((int)v, 0), (uint32_t)__builtin_amdgcn_readlane((int)v, 16)),
             max((uint32_t)__builtin_amdgcn_readlane((int)v, 32), (uint32_t)__builtin_amdgcn_readlane((int)v, 48)));
}

// (wave maximum << 32 | the slot of the lane that holds it); a wave with no
// candidate reports key 0.
__device__ inline uint64_t wave_best(uint32_t best, int bslot) {
  const uint32_t wm = wave_max_key(best);
  const int wl = __builtin_ctzll(__ballot(best == wm));
  return ((uint64_t)wm << 32) | (uint32_t)__builtin_amdgcn_readlane(bslot, wl);
}

// LDS a workgroup needs for hash_replace: the projection [D][BITS] bf16, the
// query and key rows as floats [2][D], and the exact fallback's buffers of
// the (at most two) sketching waves.
template <int D, int BITS> __host__ __device__ constexpr size_t hash_replace_lds() {
  return ((size_t)D * BITS * 2 + 2 * D * 4 + 2 * exact_lds<D>() + 15) / 16 * 16;
}

// Pre-attention replacement for one HASH unit, by the whole workgroup (every
// thread calls it with the same arguments): the sketches of the step's query
// and new key; when the cache is full (n >= B), the slot whose key sketch is
// farthest from the query's (largest Hamming distance, then the oldest
// position); token t's key and value written into that slot, or appended at
// slot n, with its sketch and position.  Logs the evicted position (-1 if
// none) when `evicted` is non-null.  `lds` is hash_replace_lds<D, BITS>()
// bytes of LDS, 16-byte aligned.  Returns the unit's new count; ends with a
// barrier, so the slot's new contents are visible to the workgroup.
template <int DT, int D, int BITS>
__device__ inline int hash_replace(const LayerCache& c, int u, int t, int B, int n, const void* q, const void* k,
                                   const void* v, int32_t* evicted, char* lds) {
  using SW = typename SkWord<BITS>::T;
  constexpr int EPL = St<DT>::EPL;
  constexpr int ES = elem_bytes<DT>();
  constexpr int LPR = D / EPL;
  __shared__ SW sk2[2];
  __shared__ uint64_t kscr[kHashNT / kWave];
  uint16_t* Ws = reinterpret_cast<uint16_t*>(lds);
  float* xs = reinterpret_cast<float*>(lds + (size_t)D * BITS * 2);   // [2][D]
  double* eb = reinterpret_cast<double*>(lds + (size_t)D * BITS * 2 + 2 * D * 4);   // [2][D + 1]
  const int tid = threadIdx.x;
  stage_proj<D, BITS>(Ws, c.proj);
  for (int i = tid; i < 2 * D; i += kHashNT)
    xs[i] = load_elem<DT>((const char*)(i < D ? q : k) + (size_t)u * D * ES, i % D);
  __syncthreads();
  // threads [0, BITS) sketch q, [BITS, 2 BITS) sketch k; one bit per lane
  if (tid < ((2 * BITS + kWave - 1) / kWave) * kWave) {   // whole waves
    const bool act = tid < 2 * BITS;
    const int r = act ? tid / BITS : 0, b = tid % BITS;
    const char* row = (const char*)(r ? k : q) + (size_t)u * D * ES;
    const int bit = sketch_bit<DT, D>(act, xs + r * D, Ws, row, c.proj, BITS, b,
                                      eb + (size_t)(tid / kWave) * (D + 1));
    const uint64_t msk = __ballot(bit != 0);
    if (act && b == 0) sk2[r] = ballot_field<BITS>(msk, tid & (kWave - 1));
  }
  __syncthreads();
  const size_t slot0 = (size_t)u * c.cap;
  int slot, ev;
  if (n >= B) {
    const SW qs = sk2[0];
    uint32_t best = 0;
    int bslot = 0;
    // PER slots per 16-byte load of sketches (4 of 32 bits, 2 of 64) and the
    // matching load of positions when the unit's first slot is aligned
    // (slot0 % PER == 0); the remainder, or every slot otherwise, one at a time
    constexpr int PER = 16 / (int)sizeof(SW);
    const SW* skp = reinterpret_cast<const SW*>(c.sk) + slot0;
    const int32_t* psp = c.pos + slot0;
    const bool vec = (slot0 % PER) == 0;
    const int nv = vec ? (n / PER) * PER : 0;
    for (int sv = tid * PER; sv < nv; sv += kHashNT * PER) {
      const uint4 a = *reinterpret_cast<const uint4*>(skp + sv);
      SW av[PER];
      int32_t pv[PER];
      __builtin_memcpy(av, &a, 16);
      if constexpr (PER == 4) {
        const int4 p = *reinterpret_cast<const int4*>(psp + sv);
        pv[0] = p.x; pv[1] = p.y; pv[2] = p.z; pv[3] = p.w;
      } else {
        const int2 p = *reinterpret_cast<const int2*>(psp + sv);
        pv[0] = p.x; pv[1] = p.y;
      }
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const uint32_t key = evict_key(popcnt(qs ^ av[j]), pv[j]);
        if (key > best) {
          best = key;
          bslot = sv + j;
        }
      }
    }
    for (int s = nv + tid; s < n; s += kHashNT) {
      const uint32_t key = evict_key(popcnt(qs ^ skp[s]), psp[s]);
      if (key > best) {
        best = key;
        bslot = s;
      }
    }
    const uint64_t wb = wave_best(best, bslot);
    if ((tid & (kWave - 1)) == 0) kscr[tid / kWave] = wb;
    __syncthreads();
    uint64_t bb = kscr[0];
#pragma unroll
    for (int w = 1; w < kHashNT / kWave; ++w) bb = kscr[w] > bb ? kscr[w] : bb;
    slot = (int)(bb & 0xFFFFFFFFu);
    ev = key_position((uint32_t)(bb >> 32));
  } else {
    slot = n;
    ev = -1;
  }
  __syncthreads();                               // every read of the old slot state is done
  if (c.q4) {
    // one element per thread: threads [0, D) the key row, [D, 2D) the value row
    constexpr int G = D / kQGroup;
    if (tid < 2 * D) {
      const bool val = tid >= D;
      const int e = tid - (val ? D : 0);
      const size_t row = slot0 + slot;
      const float x = load_elem<DT>((const char*)(val ? v : k) + (size_t)u * D * ES, e);
      q4_quantize_lane(x, e, (char*)(val ? c.V : c.K) + row * (D / 2), (val ? c.Vsc : c.Ksc) + row * G);
    }
  } else {
    char* Kd = (char*)c.K + (slot0 + slot) * D * ES;
    char* Vd = (char*)c.V + (slot0 + slot) * D * ES;
    if (tid < LPR) {
      st16(Kd + tid * EPL * ES, ld16((const char*)k + ((size_t)u * D + tid * EPL) * ES));
      st16(Vd + tid * EPL * ES, ld16((const char*)v + ((size_t)u * D + tid * EPL) * ES));
    }
  }
  if (tid == 0) {
    c.pos[slot0 + slot] = t;
    reinterpret_cast<SW*>(c.sk)[slot0 + slot] = sk2[1];
    c.S[slot0 + slot] = 0.0;
    if (slot == n) c.count[u] = n + 1;
    if (evicted) evicted[u] = ev;
  }
  __syncthreads();                               // the new row and metadata are visible
  return slot == n ? n + 1 : n;
}

}  // namespace kve
