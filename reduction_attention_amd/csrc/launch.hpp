// launch.hpp -- host-side launchers of the HIP kernels.  Arguments are
// validated by api.cpp before any launcher runs; launchers only pick a
// template instance, size the grid and enqueue on the given stream.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace rattn {

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* kv_indptr;
  void* o;         // [B, Hq, D], element type of q
  float* lse;      // [B, Hq] or nullptr
  float* o_part;   // [s, B*Hq, D]
  float* m_part;   // [s, B*Hq]
  float* l_part;   // [s, B*Hq]
  int B, Hq, Hkv, D, G;
  int s;           // split count
  int chunk;       // keys per split, ceil(max_kv_len / s)
  float scale_log2;  // scale * log2(e)
  int dtype;
  int partials_only;  // 1: every used split writes a partial, unused splits
                      // write (m, l) = (-inf, 0); 0: single-split requests are
                      // written to o / lse directly
  int uniform;        // 1: every request has max_kv_len keys (picks the
                      // workgroup shape; results do not depend on it)
  // Flat plan: the packed key rows [0, total_kv) are cut into `pieces`
  // pieces of `chunk` rows; split i of a request is its i-th piece, and s
  // bounds the splits of any request (the partial slots per row).
  int flat = 0;
  int pieces = 0;
  int64_t total_kv = 0;
};

// Multi-head latent attention decode (absorbed form): q [B, H, 576]; kv
// [total_kv, 576] (latent 512 + rotary 64 per token, shared by all heads);
// o [B, H, 512]; chunk plan of the Split operator (s chunks of `chunk` keys).
struct MlaArgs {
  const void* q;
  const void* kv;
  const int32_t* kv_indptr;
  void* o;
  float* lse;
  uint16_t* o_part;  // [s, B*H, 512] fp16, each 128-dim quarter divided by its x_part scale
  float* x_part;     // [s, B*H, 4] power-of-two scale of each quarter of the partial row
  float* m_part;     // [s, B*H]
  float* l_part;     // [s, B*H]
  int B, H;
  int s, chunk;
  float scale_log2;
  int dtype;
  int uniform;
  // Flat plan (as DecodeArgs): `pieces` pieces of `chunk` packed cache rows,
  // s bounds any request's splits.
  int flat = 0;
  int pieces = 0;
  int64_t total_kv = 0;
  // Chunk plan of the 64-head kernel: units (request, split) launched; when
  // packed (ragged lengths), at least sum over b of max(1, min(ceil(len_b /
  // chunk), s)), else s * B with unit b s + i.
  int units = 0;
  int packed = 0;
};

struct MergeArgs {
  const float* o_part;
  const float* m_part;
  const float* l_part;
  int s, rows, D;
  void* o;
  int o_dtype;
  float* lse;
  // fp16 partial rows scaled by x_part (row i of split j is
  // o_part16[j, i, :] * x_part[j, i]) in place of o_part, when not null
  const uint16_t* o_part16 = nullptr;
  const float* x_part = nullptr;
};

struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* qo_indptr;
  const int32_t* kv_indptr;
  void* o;
  float* lse;
  int B, Hq, Hkv, D, G;
  int max_q_len, max_kv_len;
  float scale_log2;
  int causal;
  int dtype;
  // Split of the key dimension (Split operator): s chunks of `chunk` keys
  // per request.  s = 1 writes o / lse; s > 1 writes, for every split i,
  // the normalised partial output as fp16 o_part[i, row, :] times the
  // power of two x_part[i, row], and its (m, l) (m in natural-log units;
  // m = -inf, l = 0 for a split without valid keys), row = (qo_indptr[b] +
  // query) * Hq + head, rows rows in all.
  int s, chunk;
  uint16_t* o_part;
  float* m_part;
  float* l_part;
  int64_t rows;
  float* x_part;
};

struct BsrArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* full_indptr;
  const int32_t* full_kblock;
  const int32_t* part_indptr;
  const int32_t* part_kblock;
  const uint64_t* part_bits;
  void* o;
  float* lse;
  int B, L, Hq, Hkv, D, G, num_blocks;
  float scale_log2;
  int dtype;
  int heads_per_mask;  // query head h uses mask h / heads_per_mask of the
                       // stacked arrays (indptr entries (num_blocks + 1) per mask)
};

// Bytes of the per-device scratch array of the entry points that allocate
// nothing, and its device address on the current device (looked up on the
// first call for each device).
constexpr size_t kScratchBytes = size_t(64) << 20;
hipError_t scratch_address(void** out);

hipError_t launch_decode(const DecodeArgs& a, hipStream_t st);
hipError_t launch_decode_partials(const DecodeArgs& a, hipStream_t st);
hipError_t launch_decode_flat(const DecodeArgs& a, hipStream_t st);
hipError_t launch_flat_ranges(const DecodeArgs& a, int32_t* ranges, hipStream_t st);
hipError_t launch_merge(const MergeArgs& a, hipStream_t st);
// MLA decode takes the many-head kernel (64 heads per workgroup) when the
// head count is a multiple of 64, the 16-head kernel otherwise.
inline bool mla_wide(int H) { return H >= 64 && H % 64 == 0; }
hipError_t launch_mla_decode(const MlaArgs& a, hipStream_t st);
hipError_t launch_split_ranges(const int32_t* kv_indptr, int B, int s, int chunk, int32_t* ranges,
                               hipStream_t st);
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t st);
int prefill_rows_per_workgroup();  // query rows one prefill workgroup covers
hipError_t launch_prefill_bsr(const BsrArgs& a, hipStream_t st);
hipError_t launch_prefill_bsr_rows(const BsrArgs& a, hipStream_t st);
hipError_t launch_bsr_decode(const int32_t* full_indptr, const int32_t* full_kblock,
                             const int32_t* part_indptr, const int32_t* part_kblock,
                             const uint64_t* part_bits, int num_blocks, uint8_t* dense,
                             hipStream_t st);

}  // namespace rattn
