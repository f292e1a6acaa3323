// Prefill scoring on the vector ALUs (any storage dtype; the path for fp32
// inputs).  Two passes over the causal score matrix s_ij = scale q_i.k_j:
//
//   rowstats: per query row i, lse_i = log sum_{j<=i} exp(s_ij) by an online
//             maximum, and optionally the prompt's attention output;
//   colsum:   per key column j, c_j = sum_{i>=j} exp(s_ij - lse_i), the
//             accumulated attention each prompt token received (H2O review
//             page, proposed method: the per-step attention statistics that
//             the greedy eviction ranks);
//   persist:  per key column j, the bits "exp(s_ij - lse_i) >= 1 / (i + 1)"
//             of the last `window` rows, bit P - 1 - i (the persistence
//             reading of the Scissorhands page).
//
// Both passes form every dot product in the same order (fmaf over d = 0..D-1
// on exact input values), so both see bit-identical logits.  lse is stored as
// a float pair (hi, lo) with hi + lo the float64 value, so exp(s - lse) keeps
// the row normaliser to float64 accuracy.
#include "common.hpp"

namespace kve {
namespace {

constexpr int kNT = 256;
constexpr int kRB = 64;   // query rows per workgroup (rowstats) / key columns (colsum)
constexpr int kKT = 32;   // keys (rowstats) / query rows (colsum) per tile

// Loads rows [r0, r0 + nrows) of a [P][D] block into LDS as float (stride D + 1);
// rows at or past P read as zero.
template <int DT, int D>
__device__ inline void stage_rows(float* dst, const char* src, int r0, int nrows, int P) {
  constexpr int EPL = St<DT>::EPL;
  constexpr int ES = elem_bytes<DT>();
  constexpr int CPR = D / EPL;
  for (int i = threadIdx.x; i < nrows * CPR; i += kNT) {
    const int r = i / CPR, cc = i % CPR;
    float f[EPL];
    if (r0 + r < P) {
      St<DT>::unpack(ld16(src + ((size_t)(r0 + r) * D + cc * EPL) * ES), f);
    } else {
#pragma unroll
      for (int j = 0; j < EPL; ++j) f[j] = 0.f;
    }
#pragma unroll
    for (int j = 0; j < EPL; ++j) dst[r * (D + 1) + cc * EPL + j] = f[j];
  }
}

template <int DT, int D>
__global__ __launch_bounds__(kNT) void rowstats_valu_kernel(Shape sh, int P, UnitList ul, const void* q,
                                                             const void* k, const void* v, float* lse,
                                                             float* out) {
  constexpr int ES = elem_bytes<DT>();
  constexpr int DS = D / 4;                  // output dims per thread
  __shared__ float Qs[kRB * (D + 1)];
  __shared__ float Ks[kKT * (D + 1)];
  __shared__ float Vs[kKT * (D + 1)];
  __shared__ float Ws[kRB * (kKT + 1)];
  __shared__ float corr_s[kRB];
  const int u = ul.ids ? ul.ids[blockIdx.y] : blockIdx.y;
  const int row0 = blockIdx.x * kRB;
  const size_t base = (size_t)u * P * D * ES;
  const char* qb = (const char*)q + base;
  const char* kb = (const char*)k + base;
  const char* vb = (const char*)v + base;
  const int tid = threadIdx.x;
  stage_rows<DT, D>(Qs, qb, row0, kRB, P);

  const int r = tid % kRB;                   // this thread's query row in the block
  const int grp = tid / kRB;                 // key subgroup (logits) / dim slice (output)
  float m = -INFINITY;                       // running max (threads tid < kRB)
  double l = 0.0;                            // running sum (threads tid < kRB)
  float o[DS];
#pragma unroll
  for (int i = 0; i < DS; ++i) o[i] = 0.f;
  const int kend = min(P, row0 + kRB);
  for (int k0 = 0; k0 < kend; k0 += kKT) {
    __syncthreads();
    stage_rows<DT, D>(Ks, kb, k0, kKT, P);
    if (out) stage_rows<DT, D>(Vs, vb, k0, kKT, P);
    __syncthreads();
    // logits: 8 keys per thread
#pragma unroll
    for (int jj = 0; jj < kKT / 4; ++jj) {
      const int j = grp * (kKT / 4) + jj;
      float s = 0.f;
      for (int e = 0; e < D; ++e) s = fmaf(Qs[r * (D + 1) + e], Ks[j * (D + 1) + e], s);
      s *= sh.scale;
      const bool ok = (k0 + j <= row0 + r) && (k0 + j < P);
      Ws[r * (kKT + 1) + j] = ok ? s : -INFINITY;
    }
    __syncthreads();
    if (tid < kRB) {
      float tmax = -INFINITY;
      for (int j = 0; j < kKT; ++j) tmax = fmaxf(tmax, Ws[tid * (kKT + 1) + j]);
      const float mn = fmaxf(m, tmax);
      const float cf = (m == -INFINITY) ? 0.f : expf(m - mn);
      float part = 0.f;
      for (int j = 0; j < kKT; ++j) {
        const float s = Ws[tid * (kKT + 1) + j];
        const float w = (s == -INFINITY) ? 0.f : expf(s - mn);
        Ws[tid * (kKT + 1) + j] = w;
        part += w;
      }
      l = l * (double)cf + (double)part;
      m = mn;
      corr_s[tid] = cf;
    }
    if (out) {
      __syncthreads();
      const float cf = corr_s[r];
#pragma unroll
      for (int i = 0; i < DS; ++i) o[i] *= cf;
      for (int j = 0; j < kKT; ++j) {
        const float w = Ws[r * (kKT + 1) + j];
#pragma unroll
        for (int i = 0; i < DS; ++i) o[i] = fmaf(w, Vs[j * (D + 1) + grp * DS + i], o[i]);
      }
    }
  }
  __syncthreads();
  if (tid < kRB && row0 + tid < P) {
    const double L = (double)m + log(l);
    const float hi = (float)L;
    lse[((size_t)u * P + row0 + tid) * 2] = hi;
    lse[((size_t)u * P + row0 + tid) * 2 + 1] = (float)(L - (double)hi);
    corr_s[tid] = (float)(1.0 / l);
  }
  if (out) {
    __syncthreads();
    if (row0 + r < P) {
      const float inv = corr_s[r];
      float* dst = out + ((size_t)u * P + row0 + r) * D + grp * DS;
#pragma unroll
      for (int i = 0; i < DS; ++i) dst[i] = o[i] * inv;
    }
  }
}

// With `mass` non-null also mass[u][j] = the part of the sum from rows >= P - rows
// (stored as float32).
template <int DT, int D>
__global__ __launch_bounds__(kNT) void colsum_valu_kernel(Shape sh, int P, UnitList ul, const void* q,
                                                           const void* k, const float* lse, double* colsum,
                                                           float* mass, int rows) {
  constexpr int ES = elem_bytes<DT>();
  __shared__ float Ks[kRB * (D + 1)];
  __shared__ float Qs[kKT * (D + 1)];
  __shared__ float Lh[kKT], Ll[kKT];
  __shared__ double part_s[kNT];
  __shared__ double mpart_s[kNT];
  const int u = ul.ids ? ul.ids[blockIdx.y] : blockIdx.y;
  const int col0 = blockIdx.x * kRB;
  const int wlo = P - rows;
  const size_t base = (size_t)u * P * D * ES;
  const int tid = threadIdx.x;
  stage_rows<DT, D>(Ks, (const char*)k + base, col0, kRB, P);
  const int jc = tid % kRB;                  // key column in the block
  const int grp = tid / kRB;                 // which 8 rows of each query tile
  double acc = 0.0, macc = 0.0;
  for (int i0 = col0; i0 < P; i0 += kKT) {
    __syncthreads();
    stage_rows<DT, D>(Qs, (const char*)q + base, i0, kKT, P);
    if (tid < kKT) {
      const size_t li = ((size_t)u * P + min(i0 + tid, P - 1)) * 2;
      Lh[tid] = lse[li];
      Ll[tid] = lse[li + 1];
    }
    __syncthreads();
    float part = 0.f, mpart = 0.f;
#pragma unroll
    for (int ii = 0; ii < kKT / 4; ++ii) {
      const int i = grp * (kKT / 4) + ii;
      float s = 0.f;
      for (int e = 0; e < D; ++e) s = fmaf(Qs[i * (D + 1) + e], Ks[jc * (D + 1) + e], s);
      s *= sh.scale;
      const bool ok = (i0 + i < P) && (i0 + i >= col0 + jc);
      if (ok) {
        const float p = expf((s - Lh[i]) - Ll[i]);
        part += p;
        if (i0 + i >= wlo) mpart += p;
      }
    }
    acc += (double)part;
    macc += (double)mpart;
  }
  part_s[tid] = acc;
  mpart_s[tid] = macc;
  __syncthreads();
  if (tid < kRB && col0 + tid < P) {
    double s = 0.0, m = 0.0;
    for (int g = 0; g < kNT / kRB; ++g) {
      s += part_s[g * kRB + tid];
      m += mpart_s[g * kRB + tid];
    }
    colsum[(size_t)u * P + col0 + tid] = s;
    if (mass) mass[(size_t)u * P + col0 + tid] = (float)m;
  }
}

template <int DT, int D>
__global__ __launch_bounds__(kNT) void persist_valu_kernel(Shape sh, int P, UnitList ul, const void* q,
                                                            const void* k, const float* lse,
                                                            const HeadMeta* meta, double* bits) {
  constexpr int ES = elem_bytes<DT>();
  __shared__ float Ks[kRB * (D + 1)];
  __shared__ float Qs[kKT * (D + 1)];
  __shared__ float Lh[kKT], Ll[kKT];
  __shared__ unsigned long long part_s[kNT];
  const int u = ul.ids ? ul.ids[blockIdx.y] : blockIdx.y;
  const int col0 = blockIdx.x * kRB;
  const size_t base = (size_t)u * P * D * ES;
  const int tid = threadIdx.x;
  const int wlo = P - meta[u].window;
  stage_rows<DT, D>(Ks, (const char*)k + base, col0, kRB, P);
  const int jc = tid % kRB;
  const int grp = tid / kRB;
  unsigned long long acc = 0;
  for (int i0 = max(col0, wlo); i0 < P; i0 += kKT) {
    __syncthreads();
    stage_rows<DT, D>(Qs, (const char*)q + base, i0, kKT, P);
    if (tid < kKT) {
      const size_t li = ((size_t)u * P + min(i0 + tid, P - 1)) * 2;
      Lh[tid] = lse[li];
      Ll[tid] = lse[li + 1];
    }
    __syncthreads();
#pragma unroll
    for (int ii = 0; ii < kKT / 4; ++ii) {
      const int i = grp * (kKT / 4) + ii;
      const int qi = i0 + i;
      float s = 0.f;
      for (int e = 0; e < D; ++e) s = fmaf(Qs[i * (D + 1) + e], Ks[jc * (D + 1) + e], s);
      s *= sh.scale;
      if (qi < P && qi >= col0 + jc) {
        // weight >= 1 / (i + 1)  <=>  s - lse >= -log(i + 1)
        const double x = ((double)s - (double)Lh[i]) - (double)Ll[i];
        if (x >= -log((double)(qi + 1))) acc |= 1ull << (P - 1 - qi);
      }
    }
  }
  part_s[tid] = acc;
  __syncthreads();
  if (tid < kRB && col0 + tid < P) {
    unsigned long long b = 0;
    for (int g = 0; g < kNT / kRB; ++g) b |= part_s[g * kRB + tid];
    reinterpret_cast<unsigned long long*>(bits)[(size_t)u * P + col0 + tid] = b;
  }
}

template <int DT, int D>
hipError_t persist_t(const Shape& sh, int P, UnitList ul, const void* q, const void* k, const float* lse,
                     const HeadMeta* meta, double* bits, hipStream_t st) {
  dim3 grid((P + kRB - 1) / kRB, ul.n);
  hipLaunchKernelGGL((persist_valu_kernel<DT, D>), grid, dim3(kNT), 0, st, sh, P, ul, q, k, lse, meta, bits);
  return hipGetLastError();
}

template <int DT, int D>
hipError_t rowstats_t(const Shape& sh, int P, UnitList ul, const void* q, const void* k, const void* v,
                      float* lse, float* out, hipStream_t st) {
  dim3 grid((P + kRB - 1) / kRB, ul.n);
  hipLaunchKernelGGL((rowstats_valu_kernel<DT, D>), grid, dim3(kNT), 0, st, sh, P, ul, q, k, v, lse, out);
  return hipGetLastError();
}

template <int DT, int D>
hipError_t colsum_t(const Shape& sh, int P, UnitList ul, const void* q, const void* k, const float* lse,
                    double* colsum, float* mass, int rows, hipStream_t st) {
  dim3 grid((P + kRB - 1) / kRB, ul.n);
  hipLaunchKernelGGL((colsum_valu_kernel<DT, D>), grid, dim3(kNT), 0, st, sh, P, ul, q, k, lse, colsum, mass,
                     rows);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_rowstats_valu(const Shape& sh, int P, UnitList ul, const void* q, const void* k,
                                        const void* v, float* lse, float* out, hipStream_t st) {
  switch (sh.dtype * 1000 + sh.d) {
    case F32 * 1000 + 64: return rowstats_t<F32, 64>(sh, P, ul, q, k, v, lse, out, st);
    case F32 * 1000 + 128: return rowstats_t<F32, 128>(sh, P, ul, q, k, v, lse, out, st);
    case F16 * 1000 + 64: return rowstats_t<F16, 64>(sh, P, ul, q, k, v, lse, out, st);
    case F16 * 1000 + 128: return rowstats_t<F16, 128>(sh, P, ul, q, k, v, lse, out, st);
    case BF16 * 1000 + 64: return rowstats_t<BF16, 64>(sh, P, ul, q, k, v, lse, out, st);
    case BF16 * 1000 + 128: return rowstats_t<BF16, 128>(sh, P, ul, q, k, v, lse, out, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_prefill_colsum_valu(const Shape& sh, int P, UnitList ul, const void* q, const void* k,
                                      const float* lse, double* colsum, hipStream_t st) {
  return launch_prefill_colsum_mass_valu(sh, P, ul, q, k, lse, colsum, nullptr, 1, st);
}

hipError_t launch_prefill_colsum_mass_valu(const Shape& sh, int P, UnitList ul, const void* q, const void* k,
                                           const float* lse, double* colsum, float* mass, int rows,
                                           hipStream_t st) {
  if (ul.n <= 0) return hipSuccess;
  switch (sh.dtype * 1000 + sh.d) {
    case F32 * 1000 + 64: return colsum_t<F32, 64>(sh, P, ul, q, k, lse, colsum, mass, rows, st);
    case F32 * 1000 + 128: return colsum_t<F32, 128>(sh, P, ul, q, k, lse, colsum, mass, rows, st);
    case F16 * 1000 + 64: return colsum_t<F16, 64>(sh, P, ul, q, k, lse, colsum, mass, rows, st);
    case F16 * 1000 + 128: return colsum_t<F16, 128>(sh, P, ul, q, k, lse, colsum, mass, rows, st);
    case BF16 * 1000 + 64: return colsum_t<BF16, 64>(sh, P, ul, q, k, lse, colsum, mass, rows, st);
    case BF16 * 1000 + 128: return colsum_t<BF16, 128>(sh, P, ul, q, k, lse, colsum, mass, rows, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace kve

namespace kve {

hipError_t launch_prefill_persist_valu(const Shape& sh, int P, UnitList ul, const void* q, const void* k,
                                       const float* lse, const HeadMeta* meta, double* bits, hipStream_t st) {
  if (ul.n <= 0) return hipSuccess;
  if (!meta) return hipErrorInvalidValue;
  switch (sh.dtype * 1000 + sh.d) {
    case F32 * 1000 + 64: return persist_t<F32, 64>(sh, P, ul, q, k, lse, meta, bits, st);
    case F32 * 1000 + 128: return persist_t<F32, 128>(sh, P, ul, q, k, lse, meta, bits, st);
    case F16 * 1000 + 64: return persist_t<F16, 64>(sh, P, ul, q, k, lse, meta, bits, st);
    case F16 * 1000 + 128: return persist_t<F16, 128>(sh, P, ul, q, k, lse, meta, bits, st);
    case BF16 * 1000 + 64: return persist_t<BF16, 64>(sh, P, ul, q, k, lse, meta, bits, st);
    case BF16 * 1000 + 128: return persist_t<BF16, 128>(sh, P, ul, q, k, lse, meta, bits, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace kve
