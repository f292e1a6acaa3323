// Fused decode step: attention over a unit's kept slots, score accumulation
// and the cache policy's replacement, one workgroup per unit.
//
// H2O review page, proposed method: each decode step's attention weights are
// the statistics that drive a greedy eviction; the lowest-scoring token
// outside the recent window leaves and the new token takes its slot.  FastGen
// review page: the same step under per-head positional policies.
//
// Layout: slot rows of d elements, 16 bytes per lane; LPR lanes cover one row
// and the workgroup covers NT / LPR rows per load wave.  Logits and then the
// unnormalised weights live in LDS (one float per slot), so the softmax is
// exact (max, then sum in float64) and the score update uses the same weights
// the output does.
#include "common.hpp"

namespace kve {
namespace {

// Compile-time tuning: rows loaded per thread before use; the register budget
// as resident waves per SIMD (0 = compiler's choice; 8 lets every workgroup of
// a 1,792-unit layer be resident at once); non-temporal K/V loads.
#ifndef KVE_DECODE_UNROLL
#define KVE_DECODE_UNROLL 2
#endif
#ifndef KVE_DECODE_WAVES_PER_EU
#define KVE_DECODE_WAVES_PER_EU 8
#endif
#ifndef KVE_DECODE_NT_LOADS
#define KVE_DECODE_NT_LOADS 1
#endif

constexpr int kNT = 256;
constexpr int kUnroll = KVE_DECODE_UNROLL;

#if KVE_DECODE_WAVES_PER_EU > 0
#define KVE_DECODE_ATTR __launch_bounds__(kNT) __attribute__((amdgpu_waves_per_eu(KVE_DECODE_WAVES_PER_EU)))
#else
#define KVE_DECODE_ATTR __launch_bounds__(kNT)
#endif

// Cached K/V rows are read once per step: optionally mark them streaming.
__device__ inline uint4 ld_kv(const void* p) {
#if KVE_DECODE_NT_LOADS
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
#else
  return ld16(p);
#endif
}

template <int DT, int D>
__global__ KVE_DECODE_ATTR void decode_fused_kernel(Shape sh, LayerCache c, DecodeIO io) {
  constexpr int EPL = St<DT>::EPL;
  constexpr int ES = elem_bytes<DT>();
  constexpr int LPR = D / EPL;
  constexpr int RPI = kNT / LPR;
  static_assert(LPR >= 4 && LPR <= 32 && kNT % LPR == 0, "row layout");

  extern __shared__ float wts[];                 // [cap + 1]
  __shared__ float red[RPI * D];
  __shared__ float fscr[kNT / kWave];
  __shared__ double dscr[kNT / kWave];
  __shared__ MinKey kscr[kNT / kWave];

  const int u = blockIdx.x;
  const int tid = threadIdx.x;
  const int col = tid % LPR;
  const int rg = tid / LPR;
  const HeadMeta m = c.meta[u % sh.heads];
  const int n = c.count[u];
  const int with_new = m.policy == HASH ? 0 : 1;  // HASH: token t is already in a slot
  const int t = io.t;
  const size_t slot0 = (size_t)u * c.cap;
  char* Kb = (char*)c.K + slot0 * D * ES;
  char* Vb = (char*)c.V + slot0 * D * ES;
  const size_t in_off = ((size_t)u * D + col * EPL) * ES;

  float qf[EPL];
  St<DT>::unpack(ld16((const char*)io.q + in_off), qf);

  // ---- logits l_j = scale * q . k_j
  for (int r0 = 0; r0 < n; r0 += RPI * kUnroll) {
    uint4 raw[kUnroll];
#pragma unroll
    for (int i = 0; i < kUnroll; ++i) {
      const int r = r0 + i * RPI + rg;
      raw[i] = r < n ? ld_kv(Kb + ((size_t)r * D + col * EPL) * ES) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < kUnroll; ++i) {
      const int r = r0 + i * RPI + rg;
      float f[EPL];
      St<DT>::unpack(raw[i], f);
      float s = 0.f;
#pragma unroll
      for (int j = 0; j < EPL; ++j) s = fmaf(qf[j], f[j], s);
      s = group_sum<LPR>(s);
      if (col == 0 && r < n) wts[r] = s * sh.scale;
    }
  }
  if (with_new && rg == 0) {
    float f[EPL];
    St<DT>::unpack(ld16((const char*)io.k + in_off), f);
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < EPL; ++j) s = fmaf(qf[j], f[j], s);
    s = group_sum<LPR>(s);
    if (col == 0) wts[n] = s * sh.scale;
  }
  __syncthreads();

  // ---- softmax over the n kept slots (+ the new token)
  const int nt = n + with_new;
  float mx = -INFINITY;
  for (int r = tid; r < nt; r += kNT) mx = fmaxf(mx, wts[r]);
  mx = block_max<kNT>(mx, fscr);
  double ls = 0.0;
  for (int r = tid; r < nt; r += kNT) {
    const float w = expf(wts[r] - mx);
    wts[r] = w;
    ls += (double)w;
  }
  const double L = block_sum<kNT>(ls, dscr);     // barriers inside: wts[] complete
  const double invL = 1.0 / L;

  // ---- output o = sum_j w_j v_j / L
  float acc[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) acc[j] = 0.f;
  for (int r0 = 0; r0 < n; r0 += RPI * kUnroll) {
    uint4 raw[kUnroll];
#pragma unroll
    for (int i = 0; i < kUnroll; ++i) {
      const int r = r0 + i * RPI + rg;
      raw[i] = r < n ? ld_kv(Vb + ((size_t)r * D + col * EPL) * ES) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < kUnroll; ++i) {
      const int r = r0 + i * RPI + rg;
      const float w = r < n ? wts[r] : 0.f;
      float f[EPL];
      St<DT>::unpack(raw[i], f);
#pragma unroll
      for (int j = 0; j < EPL; ++j) acc[j] = fmaf(w, f[j], acc[j]);
    }
  }
  if (with_new && rg == 0) {
    const float w = wts[n];
    float f[EPL];
    St<DT>::unpack(ld16((const char*)io.v + in_off), f);
#pragma unroll
    for (int j = 0; j < EPL; ++j) acc[j] = fmaf(w, f[j], acc[j]);
  }
#pragma unroll
  for (int j = 0; j < EPL; ++j) red[rg * D + col * EPL + j] = acc[j];
  __syncthreads();
  for (int i = tid; i < D; i += kNT) {
    float s = 0.f;
#pragma unroll 4
    for (int g = 0; g < RPI; ++g) s += red[g * D + i];
    io.out[(size_t)u * D + i] = (float)((double)s * invL);
  }

  // ---- the head's policy: score update, victim, in-place write
  int wslot = -1;        // slot that receives token t
  int evicted = -1;
  double s_new = 0.0;
  if (m.policy == H2O) {
    const int lim = t - m.recent;              // candidates: position <= t - recent
    MinKey best{INFINITY, INT32_MAX, INT32_MAX};
    for (int r = tid; r < n; r += kNT) {
      const double s = c.S[slot0 + r] + (double)wts[r] * invL;
      c.S[slot0 + r] = s;
      const int p = c.pos[slot0 + r];
      if (p <= lim) {
        const MinKey k{s, p, r};
        if (key_less(k, best)) best = k;
      }
    }
    s_new = (double)wts[n] * invL;
    if (tid == 0 && t <= lim) {
      const MinKey k{s_new, t, n};
      if (key_less(k, best)) best = k;
    }
    best = block_argmin<kNT>(best, kscr);      // barriers inside: S[] updates done
    if (n >= m.heavy + m.recent) {
      if (best.slot == n) {
        evicted = t;                           // the new token itself scores lowest
      } else {
        wslot = best.slot;
        evicted = best.pos;
      }
    } else {
      wslot = n;
    }
  } else if (m.policy == LOCAL) {
    if (n >= m.recent) {
      wslot = t % m.recent;                    // ring: slot of position t - W
      if (tid == 0) evicted = c.pos[slot0 + wslot];
    } else {
      wslot = n;
    }
  } else if (m.policy == FULL) {
    wslot = n;
  } else if (m.policy == SPECIAL) {
    if (token_kept(io.keep_bitmap, io.vocab, io.ids[u / sh.heads])) wslot = n;
    else evicted = t;
  }
  if (wslot >= 0) {
    __syncthreads();                           // every read of the slot is done
    if (tid < LPR) {
      st16(Kb + ((size_t)wslot * D + tid * EPL) * ES, ld16((const char*)io.k + ((size_t)u * D + tid * EPL) * ES));
      st16(Vb + ((size_t)wslot * D + tid * EPL) * ES, ld16((const char*)io.v + ((size_t)u * D + tid * EPL) * ES));
    }
    if (tid == 0) {
      c.S[slot0 + wslot] = s_new;
      c.pos[slot0 + wslot] = t;
      if (wslot == n) c.count[u] = n + 1;
    }
  }
  // HASH units log their replacement in the pre-attention kernel
  if (tid == 0 && io.evicted && m.policy != HASH) io.evicted[u] = evicted;
}

template <int DT, int D>
hipError_t launch_fused_t(const Shape& sh, const LayerCache& c, const DecodeIO& io, hipStream_t st) {
  const size_t lds = (size_t)(c.cap + 1) * sizeof(float);
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)decode_fused_kernel<DT, D>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((decode_fused_kernel<DT, D>), dim3(sh.units()), dim3(kNT), lds, st, sh, c, io);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_fused(const Shape& sh, const LayerCache& c, const DecodeIO& io, hipStream_t st) {
  switch (sh.dtype * 1000 + sh.d) {
    case F32 * 1000 + 64: return launch_fused_t<F32, 64>(sh, c, io, st);
    case F32 * 1000 + 128: return launch_fused_t<F32, 128>(sh, c, io, st);
    case F16 * 1000 + 64: return launch_fused_t<F16, 64>(sh, c, io, st);
    case F16 * 1000 + 128: return launch_fused_t<F16, 128>(sh, c, io, st);
    case BF16 * 1000 + 64: return launch_fused_t<BF16, 64>(sh, c, io, st);
    case BF16 * 1000 + 128: return launch_fused_t<BF16, 128>(sh, c, io, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace kve
