// Internal interface between the host library (kvevict.cpp) and the kernel
// launchers (*.hip).  Plain structs of device pointers; no torch types.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kve {

enum Dtype : int32_t { F32 = 0, F16 = 1, BF16 = 2 };
enum Policy : int32_t { FULL = 0, H2O = 1, LOCAL = 2, SPECIAL = 3, HASH = 4, PERSIST = 5, ADAPTIVE = 6 };

// Which token ids a unit protects (keeps for good): none, the special set,
// special or punctuation, or the SPECIAL policy's keep set.
enum IdMode : int32_t { IDS_NONE = 0, IDS_SPECIAL = 1, IDS_SPECIAL_PUNCT = 2, IDS_KEEP = 3 };

// Per-unit policy record, device-resident, one per unit of a layer (units of
// a head share it unless profiling chose per unit).
struct HeadMeta {
  int32_t policy;  // effective policy (ADAPTIVE only until the prefill chooses)
  int32_t heavy;   // H2O, PERSIST: heavy slots; HASH: budget
  int32_t recent;  // H2O, PERSIST: recent window; LOCAL: window
  int32_t cap;     // slots this unit may occupy (<= the layer's stride)
  int32_t window;  // PERSIST: steps of pivotal history (1..64)
  int32_t ids;     // IdMode: protected ids (SPECIAL: kept ids; H2O: never evicted)
  int32_t choice;  // profiled units: chosen composite 1..5 (0: not profiled)
};

// Token-id sets as device bitmaps over [0, vocab).
struct IdSets {
  const uint32_t* keep;      // SPECIAL heads' keep set
  const uint32_t* special;   // profiled heads: special tokens
  const uint32_t* punct;     // profiled heads: punctuation
  int32_t vocab;
};

// One layer's cache, carved from the workspace.
struct LayerCache {
  void* K;              // [U][cap][d] storage dtype, or [U][cap][d / 2] 4-bit code bytes (q4)
  void* V;              // [U][cap][d], likewise
  double* S;            // [U][cap] accumulated scores (H2O heads); the 64-bit
                        // pivotal histories in the same bytes (PERSIST heads)
  int32_t* pos;         // [U][cap] position per slot, -1 = empty
  void* sk;             // [U][cap] key sketches (HASH heads; 32-bit words for 16 and 32
                        // sketch bits, 64-bit words for 64), or null
  int32_t* count;       // [U] occupied slots
  int32_t* npcount;     // [U] occupied slots holding unprotected tokens (H2O units with protected ids)
  HeadMeta* meta;       // [U] (written by the prefill for profiled units)
  const uint16_t* proj; // [d][bits] bf16 projection (HASH), or null
  int32_t cap;          // slot stride per unit
  int32_t sk_bits;      // sketch width (HASH layers): 16, 32 or 64
  float* Ksc;           // [U][cap][d / 32] group scales of the 4-bit K rows (q4), else null
  float* Vsc;           // [U][cap][d / 32] group scales of the 4-bit V rows (q4), else null
  int32_t q4;           // 1: slots hold 4-bit rows (H2O and PERSIST heads only)
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
// Column sums (as launch_prefill_colsum_mfma) plus, per key, the mass the last
// `rows` prompt rows give it: mass[u][j] = sum_{i >= max(j, P - rows)} weight,
// summed in float64 and stored as float32 (one word per token: the profile).
hipError_t launch_prefill_colsum_mass_mfma(const Shape& sh, int P, UnitList units, const void* q,
                                           const void* k, const float* lse, double* colsum,
                                           float* mass, int rows, hipStream_t st);
hipError_t launch_prefill_colsum_mass_valu(const Shape& sh, int P, UnitList units, const void* q,
                                           const void* k, const float* lse, double* colsum,
                                           float* mass, int rows, hipStream_t st);
// Chooses the kept prompt positions per the unit's policy and fills the cache.
hipError_t launch_prefill_select(const Shape& sh, const LayerCache& c, int P, const double* colsum,
                                 const void* k, const void* v, const int32_t* ids, const IdSets& sets,
                                 hipStream_t st);
// Profiled units: recovered mass of each composite over the last `rows` rows,
// the first reaching `threshold` (else the full cache) becomes the unit's
// policy (meta[u] rewritten), and its kept set fills the cache.
struct Profile {
  int32_t rows;
  float threshold;
  int32_t heavy, recent;     // frequent slots and local window of the composites
};
hipError_t launch_prefill_adaptive(const Shape& sh, const LayerCache& c, UnitList units, int P,
                                   const double* colsum, const float* mass, const Profile& pf,
                                   const void* k, const void* v, const int32_t* ids, const IdSets& sets,
                                   hipStream_t st);

// ---- HashEvict
// Packed sign sketches of `n` rows of x (row stride d) under proj, per unit
// list, for rows [row0, row0 + nrows) of each unit's [P][d] block.
hipError_t launch_sketch_rows(const Shape& sh, UnitList units, const void* x, int P, int row0,
                              int nrows, const uint16_t* proj, int bits, void* out, hipStream_t st);
// Prompt replay for the listed HASH units; writes pos/sk/count, then gathers K/V.
// `max_budget` is the largest HASH budget among the listed units (LDS size).
hipError_t launch_hash_prefill(const Shape& sh, const LayerCache& c, UnitList units, int P,
                               int max_budget, const void* qsk, const void* ksk,
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
  IdSets sets;
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

// ---- static scratch (the allocation-free decode entry point)
// Size of the per-GPU static scratch array, and its device address on the
// current device (looked up once per device; thread-safe).
size_t static_scratch_bytes();
hipError_t static_scratch_address(void** out);

// ---- measurement
// Reads `bytes` (a multiple of 16, 16-byte aligned) of src with the decode
// kernels' 16-byte non-temporal loads; writes nothing in practice (sink is
// written only if the XOR of a workgroup's bytes equals a fixed constant).
hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t st);


}  // namespace kve
