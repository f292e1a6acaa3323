// Internal interface between the host library (kvevict.cpp) and the kernel
// launchers (*.hip).  Plain structs of device pointers; no torch types.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kve {

enum Dtype : int32_t { F32 = 0, F16 = 1, BF16 = 2 };
enum Policy : int32_t { FULL = 0, H2O = 1, LOCAL = 2, SPECIAL = 3, HASH = 4, PERSIST = 5 };

// Per-head policy record, device-resident, one per head of a layer.
struct HeadMeta {
  int32_t policy;
  int32_t heavy;   // H2O, PERSIST: heavy slots; HASH: budget
  int32_t recent;  // H2O, PERSIST: recent window; LOCAL: window
  int32_t cap;     // slots this head may occupy (<= the layer's stride)
  int32_t window;  // PERSIST: steps of pivotal history (1..64)
};

// One layer's cache, carved from the workspace.
struct LayerCache {
  void* K;              // [U][cap][d] storage dtype
  void* V;              // [U][cap][d]
  double* S;            // [U][cap] accumulated scores (H2O heads); the 64-bit
                        // pivotal histories in the same bytes (PERSIST heads)
  int32_t* pos;         // [U][cap] position per slot, -1 = empty
  uint32_t* sk;         // [U][cap] key sketches (HASH heads), or null
  int32_t* count;       // [U] occupied slots
  const HeadMeta* meta; // [heads]
  const uint16_t* proj; // [d][bits] bf16 projection (HASH), or null
  int32_t cap;          // slot stride per unit
};

struct Shape {
  int32_t batch, heads, d, dtype;
  float scale;
  int32_t units() const { return batch * heads; }
};

// Unit lists: device int32 arrays of unit indices; null means all units.
struct UnitList {
  const int32_t* ids;
  int32_t n;
};

// ---- prefill
// lse[u][i] = log sum_{j<=i} exp(scale q_i.k_j) for the listed units, stored
// as a float pair (hi, lo) whose sum is the float64 value; when `out` is
// non-null also out[u][i][:] = causal attention output (fp32).
hipError_t launch_prefill_rowstats_valu(const Shape& sh, int P, UnitList units, const void* q,
                                        const void* k, const void* v, float* lse, float* out,
                                        hipStream_t st);
// colsum[u][j] = sum_{i>=j} exp(scale q_i.k_j - lse[u][i]), float64.
hipError_t launch_prefill_colsum_valu(const Shape& sh, int P, UnitList units, const void* q,
                                      const void* k, const float* lse, double* colsum,
                                      hipStream_t st);
// The same two passes on the matrix cores (16-bit dtypes only).  rowstats
// covers the 128-query blocks that hold rows >= q_from (0: every row).
hipError_t launch_prefill_rowstats_mfma(const Shape& sh, int P, UnitList units, const void* q,
                                        const void* k, float* lse, int q_from, hipStream_t st);
// Row statistics and the causal attention output out[u][i][:] (fp32) on the
// matrix cores (16-bit dtypes only).
hipError_t launch_prefill_attend_mfma(const Shape& sh, int P, UnitList units, const void* q,
                                      const void* k, const void* v, float* lse, float* out,
                                      hipStream_t st);
hipError_t launch_prefill_colsum_mfma(const Shape& sh, int P, UnitList units, const void* q,
                                      const void* k, const float* lse, double* colsum,
                                      hipStream_t st);
// Pivotal histories of the prompt for the listed PERSIST units, into the
// colsum array as 64-bit patterns: bit P - 1 - i of key j is set iff row i,
// with max(j, P - window) <= i < P, gives key j a weight >= 1 / (i + 1).
// Needs lse for those rows.  meta: the layer's head table (window per head).
hipError_t launch_prefill_persist_mfma(const Shape& sh, int P, UnitList units, const void* q,
                                       const void* k, const float* lse, const HeadMeta* meta,
                                       double* bits, hipStream_t st);
hipError_t launch_prefill_persist_valu(const Shape& sh, int P, UnitList units, const void* q,
                                       const void* k, const float* lse, const HeadMeta* meta,
                                       double* bits, hipStream_t st);
// Chooses the kept prompt positions per the head's policy and fills the cache.
hipError_t launch_prefill_select(const Shape& sh, const LayerCache& c, int P, const double* colsum,
                                 const void* k, const void* v, const int32_t* ids,
                                 const uint32_t* keep_bitmap, int32_t vocab, hipStream_t st);

// ---- HashEvict
// Packed sign sketches of `n` rows of x (row stride d) under proj, per unit
// list, for rows [row0, row0 + nrows) of each unit's [P][d] block.
hipError_t launch_sketch_rows(const Shape& sh, UnitList units, const void* x, int P, int row0,
                              int nrows, const uint16_t* proj, uint32_t* out, hipStream_t st);
// Prompt replay for the listed HASH units; writes pos/sk/count, then gathers K/V.
// `max_budget` is the largest HASH budget among the listed units (LDS size).
hipError_t launch_hash_prefill(const Shape& sh, const LayerCache& c, UnitList units, int P,
                               int max_budget, const uint32_t* qsk, const uint32_t* ksk,
                               const void* k, const void* v, hipStream_t st);
// Decode: replacement before attention for the listed HASH units.
hipError_t launch_hash_evict(const Shape& sh, const LayerCache& c, UnitList units, int t,
                             const void* q, const void* k, const void* v, int32_t* evicted,
                             hipStream_t st);

// ---- decode
struct DecodeIO {
  const void* q;            // [U][d]
  const void* k;            // [U][d]
  const void* v;            // [U][d]
  const int32_t* ids;       // [batch] or null
  const uint32_t* keep_bitmap;
  int32_t vocab;
  float* out;               // [U][d]
  int32_t* evicted;         // [U] or null
  int32_t t;                // position of the new token
};

// Scratch of the split decode: per-chunk partials [U][max_chunks][d + 2]
// (unnormalised output, chunk maximum, chunk sum) and raw logits [U][cap].
constexpr int kMaxChunks = 64;
struct SplitScratch {
  float* part;
  float* logits;
  int32_t chunk;        // slots per chunk
  int32_t max_chunks;   // ceil(cap / chunk), <= kMaxChunks
};

// Attention + score update + policy step for every unit of the layer: one
// workgroup per unit when sp is null, else partials over (unit, chunk) then a
// per-unit combine.
hipError_t launch_decode(const Shape& sh, const LayerCache& c, const DecodeIO& io,
                         const SplitScratch* sp, hipStream_t st);


}  // namespace kve
