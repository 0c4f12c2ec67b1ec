// api.cpp -- the C ABI declared in include/attn.h: argument validation,
// status reporting, the split-count rule, workspace sizing, the host-side
// BSR encoder, and dispatch to the kernel launchers.  No HIP call is made
// before an argument check has passed.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/attn.h"
#include "launch.hpp"

namespace {

thread_local std::string g_last_error;

attn_status_t fail(attn_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

attn_status_t ok() {
  g_last_error.clear();
  return ATTN_OK;
}

attn_status_t hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(ATTN_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool valid_dtype(int dt) { return dt == ATTN_F32 || dt == ATTN_BF16 || dt == ATTN_F16; }

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kMaxSplits = 256;
constexpr int kMaxGroup = 16;
constexpr int kMaxPieces = 65535;
static_assert(rattn::kScratchBytes == ATTN_NOALLOC_SCRATCH_BYTES,
              "scratch array size differs from the header's");

}  // namespace

extern "C" {

const char* attn_status_string(attn_status_t s) {
  switch (s) {
    case ATTN_OK: return "ATTN_OK";
    case ATTN_EINVAL: return "ATTN_EINVAL: invalid argument";
    case ATTN_EUNSUPPORTED: return "ATTN_EUNSUPPORTED: unsupported configuration";
    case ATTN_EWORKSPACE: return "ATTN_EWORKSPACE: workspace missing or too small";
    case ATTN_EHIP: return "ATTN_EHIP: HIP runtime error";
  }
  return "unknown attn status";
}

const char* attn_last_error(void) { return g_last_error.c_str(); }

int attn_device_cu_count(void) {
  static std::once_flag once;
  static int cus = 256;
  std::call_once(once, [] {
    int dev = 0;
    hipDeviceProp_t prop;
    if (hipGetDevice(&dev) == hipSuccess && hipGetDeviceProperties(&prop, dev) == hipSuccess &&
        prop.multiProcessorCount > 0)
      cus = prop.multiProcessorCount;
    else
      (void)hipGetLastError();
  });
  return cus;
}

// Workspace layout: o_part [s, B*Hq, D], m_part [s, B*Hq], l_part [s, B*Hq] (fp32).
size_t attn_decode_workspace_bytes(int B, int Hq, int D, int num_splits) {
  if (B <= 0 || Hq <= 0 || D <= 0 || num_splits <= 0 || num_splits > kMaxSplits) return 0;
  const size_t rows = size_t(B) * size_t(Hq);
  const size_t bytes = size_t(num_splits) * rows * (size_t(D) + 2) * sizeof(float);
  return (bytes + 255) & ~size_t(255);
}

// Equal or nearly equal lengths: the mean length is at least 15/16 of the
// longest (equal lengths are the exact case).  Nearly all the keys then sit
// in full chunks, so the equal-length shapes, whose workgroups each own a
// whole chunk, stay balanced; they are correct for any lengths (a chunk
// past a request's end is empty), only slower where lengths spread widely.
static int uniform_lengths(int B, int max_kv_len, long long total_kv) {
  if (B <= 0 || max_kv_len <= 0) return 0;
  return 16 * total_kv >= 15LL * B * max_kv_len ? 1 : 0;
}

int attn_decode_choose_splits(int B, int Hq, int Hkv, int D, long long total_kv, int max_kv_len) {
  (void)Hq;
  (void)D;
  if (B <= 0 || Hkv <= 0 || max_kv_len <= 256 || total_kv <= 0) return 1;
  const long long cus = attn_device_cu_count();
  long long c = 1;
  while (c < max_kv_len) c <<= 1;  // one split per request at most
  if (uniform_lengths(B, max_kv_len, total_kv)) {
    // Equal (or nearly equal) lengths: workgroups of up to four KV heads,
    // each wave streaming a whole chunk.  Largest power-of-two chunk >= 256
    // that gives every compute unit a workgroup.
    const int hpw = Hkv >= 4 ? 4 : Hkv >= 2 ? 2 : 1;
    const long long groups = (Hkv + hpw - 1) / hpw;
    while (c > 256 && groups * B * ((max_kv_len + c - 1) / c) < cus) c >>= 1;
  } else {
    // Ragged lengths: one KV head per workgroup, four waves per chunk.  Aim
    // for four (head, chunk) workgroups per compute unit, so that smaller
    // chunks even out the uneven last chunks of the requests.
    while (c > 256) {
      const long long wgs = (long long)Hkv * ((total_kv + c - 1) / c + B / 2);
      if (wgs >= 4 * cus) break;
      c >>= 1;
    }
  }
  long long s = (max_kv_len + c - 1) / c;
  if (s < 1) s = 1;
  if (s > kMaxSplits) s = kMaxSplits;
  return int(s);
}

attn_status_t attn_merge_lse(const float* o_part, const float* m_part, const float* l_part,
                             int num_splits, int rows, int D, void* o, int o_dtype, float* lse,
                             void* hip_stream) {
  if (!o_part || !m_part || !l_part || !o) return fail(ATTN_EINVAL, "merge: null pointer");
  if (num_splits < 1 || num_splits > kMaxSplits)
    return fail(ATTN_EINVAL, "merge: num_splits %d outside [1, %d]", num_splits, kMaxSplits);
  if (rows < 0) return fail(ATTN_EINVAL, "merge: rows %d < 0", rows);
  if (rows > (1 << 30)) return fail(ATTN_EUNSUPPORTED, "merge: rows above 2^30");
  if (D != 64 && D != 128) return fail(ATTN_EUNSUPPORTED, "merge: D = %d (supported: 64, 128)", D);
  if (!valid_dtype(o_dtype)) return fail(ATTN_EUNSUPPORTED, "merge: o_dtype %d", o_dtype);
  rattn::MergeArgs a{o_part, m_part, l_part, num_splits, rows, D, o, o_dtype, lse};
  return hip_status(rattn::launch_merge(a, static_cast<hipStream_t>(hip_stream)), "merge launch");
}

static attn_status_t check_decode(const void* q, const void* k, const void* v,
                                  const int32_t* kv_indptr, int B, int Hq, int Hkv, int D,
                                  int max_kv_len, long long total_kv, float scale, int num_splits,
                                  int dtype) {
  if (!q || !k || !v || !kv_indptr) return fail(ATTN_EINVAL, "decode: null pointer");
  if (B < 1 || Hq < 1 || Hkv < 1) return fail(ATTN_EINVAL, "decode: B, Hq, Hkv must be >= 1");
  if (B > 65535 || Hkv > 65535) return fail(ATTN_EUNSUPPORTED, "decode: B or Hkv above 65535");
  if (Hq % Hkv) return fail(ATTN_EINVAL, "decode: Hq %d not a multiple of Hkv %d", Hq, Hkv);
  if (Hq / Hkv > kMaxGroup)
    return fail(ATTN_EUNSUPPORTED, "decode: group size %d above %d", Hq / Hkv, kMaxGroup);
  if ((long long)B * Hq > (1LL << 30)) return fail(ATTN_EUNSUPPORTED, "decode: B * Hq above 2^30");
  if (D != 64 && D != 128) return fail(ATTN_EUNSUPPORTED, "decode: D = %d (supported: 64, 128)", D);
  if (!valid_dtype(dtype)) return fail(ATTN_EUNSUPPORTED, "decode: dtype %d", dtype);
  if (max_kv_len < 0 || total_kv < 0) return fail(ATTN_EINVAL, "decode: negative length");
  if ((long long)max_kv_len > total_kv)
    return fail(ATTN_EINVAL, "decode: max_kv_len %d exceeds total_kv %lld", max_kv_len, total_kv);
  if (!std::isfinite(scale)) return fail(ATTN_EINVAL, "decode: scale is not finite");
  if (num_splits < 0 || num_splits > kMaxSplits)
    return fail(ATTN_EINVAL, "decode: num_splits %d outside [0, %d]", num_splits, kMaxSplits);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v))
    return fail(ATTN_EINVAL, "decode: q, k, v must be 16-byte aligned");
  return ATTN_OK;
}

// The two kernels of attn_decode_splitkv with s splits, the partials in
// `workspace` (validated by the caller).
static attn_status_t decode_run(const void* q, const void* k, const void* v,
                                const int32_t* kv_indptr, void* o, float* lse, int B, int Hq,
                                int Hkv, int D, int max_kv_len, long long total_kv, float scale,
                                int s, int dtype, void* workspace, void* hip_stream) {
  const int chunk = max_kv_len > 0 ? (max_kv_len + s - 1) / s : 0;
  const size_t rows = size_t(B) * Hq;
  float* ws = static_cast<float*>(workspace);
  rattn::DecodeArgs a{q, k, v, kv_indptr, o, lse, ws, ws + size_t(s) * rows * D,
                      ws + size_t(s) * rows * D + size_t(s) * rows,
                      B, Hq, Hkv, D, Hq / Hkv, s, chunk, scale * kLog2e, dtype, 0,
                      uniform_lengths(B, max_kv_len, total_kv)};
  return hip_status(rattn::launch_decode(a, static_cast<hipStream_t>(hip_stream)), "decode launch");
}

attn_status_t attn_decode_splitkv(const void* q, const void* k, const void* v,
                                  const int32_t* kv_indptr, void* o, float* lse, int B, int Hq,
                                  int Hkv, int D, int max_kv_len, long long total_kv, float scale,
                                  int num_splits, int dtype, void* workspace,
                                  size_t workspace_bytes, void* hip_stream) {
  attn_status_t cs = check_decode(q, k, v, kv_indptr, B, Hq, Hkv, D, max_kv_len, total_kv, scale,
                                  num_splits, dtype);
  if (cs != ATTN_OK) return cs;
  if (!o) return fail(ATTN_EINVAL, "decode: null output");
  if (!aligned16(o)) return fail(ATTN_EINVAL, "decode: o must be 16-byte aligned");
  const int s = num_splits ? num_splits
                           : attn_decode_choose_splits(B, Hq, Hkv, D, total_kv, max_kv_len);
  const size_t need = attn_decode_workspace_bytes(B, Hq, D, s);
  if (!workspace || workspace_bytes < need)
    return fail(ATTN_EWORKSPACE, "decode: workspace needs %zu bytes, got %zu", need,
                workspace ? workspace_bytes : size_t(0));
  if (!aligned16(workspace)) return fail(ATTN_EINVAL, "decode: workspace must be 16-byte aligned");
  return decode_run(q, k, v, kv_indptr, o, lse, B, Hq, Hkv, D, max_kv_len, total_kv, scale, s,
                    dtype, workspace, hip_stream);
}

attn_status_t attn_decode_splitkv_noalloc(const void* q, const void* k, const void* v,
                                          const int32_t* kv_indptr, void* o, float* lse, int B,
                                          int Hq, int Hkv, int D, int max_kv_len,
                                          long long total_kv, float scale, int num_splits,
                                          int dtype, void* hip_stream) {
  attn_status_t cs = check_decode(q, k, v, kv_indptr, B, Hq, Hkv, D, max_kv_len, total_kv, scale,
                                  num_splits, dtype);
  if (cs != ATTN_OK) return cs;
  if (!o) return fail(ATTN_EINVAL, "decode_noalloc: null output");
  if (!aligned16(o)) return fail(ATTN_EINVAL, "decode_noalloc: o must be 16-byte aligned");
  const int s = num_splits ? num_splits
                           : attn_decode_choose_splits(B, Hq, Hkv, D, total_kv, max_kv_len);
  const size_t need = attn_decode_workspace_bytes(B, Hq, D, s);
  if (need > rattn::kScratchBytes)
    return fail(ATTN_EWORKSPACE,
                "decode_noalloc: %d splits need %zu bytes of partials, above the %zu-byte "
                "scratch array (use attn_decode_splitkv with a workspace, or fewer splits)",
                s, need, size_t(rattn::kScratchBytes));
  void* scratch = nullptr;
  attn_status_t hs = hip_status(rattn::scratch_address(&scratch), "decode_noalloc: scratch address");
  if (hs != ATTN_OK) return hs;
  return decode_run(q, k, v, kv_indptr, o, lse, B, Hq, Hkv, D, max_kv_len, total_kv, scale, s,
                    dtype, scratch, hip_stream);
}

attn_status_t attn_decode_partials(const void* q, const void* k, const void* v,
                                   const int32_t* kv_indptr, int B, int Hq, int Hkv, int D,
                                   int max_kv_len, long long total_kv, float scale, int num_splits,
                                   int dtype, float* o_part, float* m_part, float* l_part,
                                   void* hip_stream) {
  attn_status_t cs = check_decode(q, k, v, kv_indptr, B, Hq, Hkv, D, max_kv_len, total_kv, scale,
                                  num_splits, dtype);
  if (cs != ATTN_OK) return cs;
  if (num_splits < 1) return fail(ATTN_EINVAL, "decode_partials: num_splits must be >= 1");
  if (!o_part || !m_part || !l_part) return fail(ATTN_EINVAL, "decode_partials: null output");
  const int chunk = max_kv_len > 0 ? (max_kv_len + num_splits - 1) / num_splits : 0;
  rattn::DecodeArgs a{q, k, v, kv_indptr, nullptr, nullptr, o_part, m_part, l_part,
                      B, Hq, Hkv, D, Hq / Hkv, num_splits, chunk, scale * kLog2e, dtype, 1,
                      uniform_lengths(B, max_kv_len, total_kv)};
  return hip_status(rattn::launch_decode_partials(a, static_cast<hipStream_t>(hip_stream)),
                    "decode_partials launch");
}

// ---- multi-head latent attention decode ---------------------------------------

// MLA workspace layout: o_part [s, B*H, 512] (fp16 bits), then the fp32
// arrays x_part [s, B*H, 4] (scale of each 128-dim quarter of a partial
// row), m_part [s, B*H] and l_part [s, B*H].
static size_t mla_workspace_raw(size_t s, size_t rows) {
  return s * rows * (512 * sizeof(uint16_t) + (4 + 2) * sizeof(float));
}
static void mla_workspace_split(void* workspace, size_t s, size_t rows, rattn::MlaArgs& a) {
  if (!workspace) return;
  a.o_part = static_cast<uint16_t*>(workspace);
  a.x_part = reinterpret_cast<float*>(a.o_part + s * rows * 512);
  a.m_part = a.x_part + s * rows * 4;
  a.l_part = a.m_part + s * rows;
}

size_t attn_mla_decode_workspace_bytes(int B, int H, int num_splits) {
  if (B <= 0 || H <= 0 || num_splits <= 0 || num_splits > kMaxSplits) return 0;
  const size_t bytes = mla_workspace_raw(size_t(num_splits), size_t(B) * size_t(H));
  return (bytes + 255) & ~size_t(255);
}

int attn_mla_decode_choose_splits(int B, int H, long long total_kv, int max_kv_len) {
  if (B <= 0 || H <= 0 || max_kv_len <= 256 || total_kv <= 0) return 1;
  // hg workgroups (16 heads each, 64 for the many-head kernel) per chunk.
  const long long cus = attn_device_cu_count();
  const bool wide = rattn::mla_wide(H);
  const long long hg = wide ? H / 64 : (H + 15) / 16;
  const bool uniform = uniform_lengths(B, max_kv_len, total_kv) != 0;  // or nearly equal
  if (wide && !uniform) {
    // Packed units (only the chunks a request has; about total_kv / c + B / 2
    // of them, a request's last chunk being half full on average), hg
    // workgroups each and one workgroup per compute unit (the kernel holds
    // all of its LDS): the shortest chunk, at least 256 keys, whose units
    // fill k rounds of 95% of the compute units, k the fewest rounds that
    // leave half a round for chunks beside the requests' last ones.  The
    // units of an XCD that do not fit its compute units wait for a whole
    // chunk, so s is rounded down: the chunk ceil(max_kv_len / s) is then
    // no shorter than c.
    const double slots = 0.95 * double(cus) / double(hg);
    const double k = std::ceil((B / 2.0 + slots / 2.0) / slots);
    const double room = k * slots - B / 2.0;
    const long long c = std::max(256LL, (long long)std::ceil(double(total_kv) / room));
    long long s = max_kv_len / c;
    // B * s bounds the unit count exactly, so any s with B * s units at most
    // one per compute unit is safe whatever the lengths, and may exceed the
    // estimate's s where it counts the last chunks as half full.
    const long long s_exact = std::min(cus / hg / B, (long long)max_kv_len / 256);
    if (s_exact > s) s = s_exact;
    if (s < 1) s = 1;
    if (s > kMaxSplits) s = kMaxSplits;
    return int(s);
  }
  // Equal (or nearly equal) lengths: the largest power-of-two chunk >= 256
  // keys that gives every compute unit a workgroup.  Ragged, 16-head
  // kernel: chunks counted as total/c + B/2, two workgroups per compute
  // unit, and an odd s: its workgroups are dealt to the eight XCDs round
  // robin by (request, split) slot, and with s a multiple of eight the first
  // splits (present in every request) would all land on the same XCDs while
  // the last ones (mostly empty) land on the others.
  long long c = 1;
  while (c < max_kv_len) c <<= 1;
  while (c > 256) {
    const long long chunks = uniform ? B * ((max_kv_len + c - 1) / c) : (total_kv + c - 1) / c + B / 2;
    if (hg * chunks >= (uniform ? 1 : 2) * cus) break;
    c >>= 1;
  }
  long long s = (max_kv_len + c - 1) / c;
  if (!uniform && s > 1 && s % 2 == 0) s += 1;
  if (s < 1) s = 1;
  if (s > kMaxSplits) s = kMaxSplits;
  return int(s);
}

attn_status_t attn_mla_decode(const void* q, const void* kv, const int32_t* kv_indptr, void* o,
                              float* lse, int B, int H, int Dc, int Dr, int max_kv_len,
                              long long total_kv, float scale, int num_splits, int dtype,
                              void* workspace, size_t workspace_bytes, void* hip_stream) {
  if (!q || !kv || !kv_indptr || !o) return fail(ATTN_EINVAL, "mla_decode: null pointer");
  if (B < 1 || H < 1) return fail(ATTN_EINVAL, "mla_decode: B and H must be >= 1");
  if ((long long)B * H > (1LL << 30)) return fail(ATTN_EUNSUPPORTED, "mla_decode: B * H above 2^30");
  if (Dc != 512 || Dr != 64)
    return fail(ATTN_EUNSUPPORTED, "mla_decode: latent/rotary widths %d/%d (supported: 512/64)", Dc,
                Dr);
  if (dtype != ATTN_BF16 && dtype != ATTN_F16)
    return fail(ATTN_EUNSUPPORTED, "mla_decode: dtype %d (16-bit only)", dtype);
  if (max_kv_len < 0 || total_kv < 0) return fail(ATTN_EINVAL, "mla_decode: negative length");
  if ((long long)max_kv_len > total_kv)
    return fail(ATTN_EINVAL, "mla_decode: max_kv_len %d exceeds total_kv %lld", max_kv_len, total_kv);
  if (!std::isfinite(scale)) return fail(ATTN_EINVAL, "mla_decode: scale is not finite");
  if (num_splits < 0 || num_splits > kMaxSplits)
    return fail(ATTN_EINVAL, "mla_decode: num_splits %d outside [0, %d]", num_splits, kMaxSplits);
  if (!aligned16(q) || !aligned16(kv) || !aligned16(o))
    return fail(ATTN_EINVAL, "mla_decode: q, kv, o must be 16-byte aligned");
  const int s = num_splits ? num_splits : attn_mla_decode_choose_splits(B, H, total_kv, max_kv_len);
  if ((long long)s * B > (1LL << 27)) return fail(ATTN_EUNSUPPORTED, "mla_decode: s * B too large");
  const size_t need = attn_mla_decode_workspace_bytes(B, H, s);
  if (s > 1 && (!workspace || workspace_bytes < need))
    return fail(ATTN_EWORKSPACE, "mla_decode: workspace needs %zu bytes, got %zu", need,
                workspace ? workspace_bytes : size_t(0));
  if (s > 1 && !aligned16(workspace))
    return fail(ATTN_EINVAL, "mla_decode: workspace must be 16-byte aligned");
  const size_t rows = size_t(B) * H;
  rattn::MlaArgs a{q, kv, kv_indptr, o, lse, nullptr, nullptr, nullptr, nullptr,
                   B, H, s, max_kv_len > 0 ? (max_kv_len + s - 1) / s : 1, scale * kLog2e, dtype,
                   uniform_lengths(B, max_kv_len, total_kv)};
  if (s > 1) mla_workspace_split(workspace, size_t(s), rows, a);
  a.total_kv = total_kv;
  // the 64-head kernel's units: for ragged lengths packed (request b owns
  // max(1, min(ceil(len_b / c), s)) <= len_b / c + 1 of them), else all
  // s * B (request b, split i at b s + i: no lookup at start-up)
  a.packed = a.uniform ? 0 : 1;
  a.units = a.packed ? int(std::min((long long)s * B, (total_kv + a.chunk - 1) / a.chunk + B))
                     : s * B;
  return hip_status(rattn::launch_mla_decode(a, static_cast<hipStream_t>(hip_stream)),
                    "mla_decode launch");
}

// ---- MLA decode, flat plan ------------------------------------------------------

static long long flat_piece_len(long long total_kv, int P) {
  return total_kv > 0 ? (total_kv + P - 1) / P : 0;
}

int attn_mla_decode_flat_pieces(int B, int H, long long total_kv) {
  (void)B;
  if (H <= 0 || H % 64 || total_kv <= 0) return 1;
  // one many-head workgroup (64 heads, all of a compute unit's LDS) per
  // compute unit: CUs / (H / 64) pieces, none shorter than 256 keys
  long long P = attn_device_cu_count() / (H / 64);
  const long long cap = (total_kv + 255) / 256;
  if (P > cap) P = cap;
  if (P < 1) P = 1;
  if (P > kMaxPieces) P = kMaxPieces;
  return int(P);
}

size_t attn_mla_decode_flat_workspace_bytes(int B, int H, int max_kv_len, long long total_kv,
                                            int num_pieces) {
  const int s = attn_decode_flat_max_splits(max_kv_len, total_kv, num_pieces);
  if (B <= 0 || H <= 0 || s <= 0) return 0;
  const size_t bytes = mla_workspace_raw(size_t(s), size_t(B) * size_t(H));
  return (bytes + 255) & ~size_t(255);
}

attn_status_t attn_mla_decode_flat(const void* q, const void* kv, const int32_t* kv_indptr, void* o,
                                   float* lse, int B, int H, int Dc, int Dr, int max_kv_len,
                                   long long total_kv, float scale, int num_pieces, int dtype,
                                   void* workspace, size_t workspace_bytes, void* hip_stream) {
  if (!q || !kv || !kv_indptr || !o) return fail(ATTN_EINVAL, "mla_decode_flat: null pointer");
  if (B < 1 || H < 1) return fail(ATTN_EINVAL, "mla_decode_flat: B and H must be >= 1");
  if (H % 64)
    return fail(ATTN_EUNSUPPORTED, "mla_decode_flat: H = %d is not a multiple of 64", H);
  if ((long long)B * H > (1LL << 30))
    return fail(ATTN_EUNSUPPORTED, "mla_decode_flat: B * H above 2^30");
  if (Dc != 512 || Dr != 64)
    return fail(ATTN_EUNSUPPORTED, "mla_decode_flat: latent/rotary widths %d/%d (supported: 512/64)",
                Dc, Dr);
  if (dtype != ATTN_BF16 && dtype != ATTN_F16)
    return fail(ATTN_EUNSUPPORTED, "mla_decode_flat: dtype %d (16-bit only)", dtype);
  if (max_kv_len < 0 || total_kv < 0) return fail(ATTN_EINVAL, "mla_decode_flat: negative length");
  if ((long long)max_kv_len > total_kv)
    return fail(ATTN_EINVAL, "mla_decode_flat: max_kv_len %d exceeds total_kv %lld", max_kv_len,
                total_kv);
  if (total_kv > 0x7fffffffLL)
    return fail(ATTN_EUNSUPPORTED, "mla_decode_flat: total_kv above 2^31 - 1");
  if (!std::isfinite(scale)) return fail(ATTN_EINVAL, "mla_decode_flat: scale is not finite");
  if (num_pieces < 0 || num_pieces > kMaxPieces)
    return fail(ATTN_EINVAL, "mla_decode_flat: num_pieces %d outside [0, %d]", num_pieces, kMaxPieces);
  if (!aligned16(q) || !aligned16(kv) || !aligned16(o))
    return fail(ATTN_EINVAL, "mla_decode_flat: q, kv, o must be 16-byte aligned");
  const int P = num_pieces ? num_pieces : attn_mla_decode_flat_pieces(B, H, total_kv);
  const int s = attn_decode_flat_max_splits(max_kv_len, total_kv, P);
  const size_t need = attn_mla_decode_flat_workspace_bytes(B, H, max_kv_len, total_kv, P);
  if (!workspace || workspace_bytes < need)
    return fail(ATTN_EWORKSPACE, "mla_decode_flat: workspace needs %zu bytes, got %zu", need,
                workspace ? workspace_bytes : size_t(0));
  if (!aligned16(workspace))
    return fail(ATTN_EINVAL, "mla_decode_flat: workspace must be 16-byte aligned");
  const size_t rows = size_t(B) * H;
  rattn::MlaArgs a{q, kv, kv_indptr, o, lse, nullptr, nullptr, nullptr, nullptr, B, H, s,
                   int(flat_piece_len(total_kv, P)),
                   scale * kLog2e, dtype, 0};
  mla_workspace_split(workspace, size_t(s), rows, a);
  a.flat = 1;
  a.pieces = P;
  a.total_kv = total_kv;
  return hip_status(rattn::launch_mla_decode(a, static_cast<hipStream_t>(hip_stream)),
                    "mla_decode_flat launch");
}

// ---- flat split plan -------------------------------------------------------

int attn_decode_flat_pieces(int B, int Hq, int Hkv, int D, long long total_kv) {
  (void)B;
  (void)Hq;
  (void)D;
  if (Hkv <= 0 || total_kv <= 0) return 1;
  // Workgroups of up to four KV heads side by side; enough pieces for four
  // waves per compute unit, all resident at once (a sweep on MI355X over
  // 128..384 pieces and 1..8 heads per workgroup peaked there), and no
  // piece shorter than 256 keys.
  const int hpw = Hkv >= 4 ? 4 : Hkv >= 2 ? 2 : 1;
  const long long groups = (Hkv + hpw - 1) / hpw;
  long long P = (4LL * attn_device_cu_count() + groups * hpw - 1) / (groups * hpw);
  const long long cap = (total_kv + 255) / 256;
  if (P > cap) P = cap;
  if (P < 1) P = 1;
  if (P > kMaxPieces) P = kMaxPieces;
  return int(P);
}

int attn_decode_flat_max_splits(int max_kv_len, long long total_kv, int num_pieces) {
  if (num_pieces < 1 || total_kv < 0 || max_kv_len < 0) return 0;
  const long long c = flat_piece_len(total_kv, num_pieces);
  if (c == 0 || max_kv_len == 0) return 1;
  const long long s = (max_kv_len - 1 + c - 1) / c + 1;
  return int(s < num_pieces ? s : num_pieces);
}

size_t attn_decode_flat_workspace_bytes(int B, int Hq, int D, int max_kv_len, long long total_kv,
                                        int num_pieces) {
  const int s = attn_decode_flat_max_splits(max_kv_len, total_kv, num_pieces);
  if (B <= 0 || Hq <= 0 || D <= 0 || s <= 0) return 0;
  const size_t bytes = size_t(s) * size_t(B) * size_t(Hq) * (size_t(D) + 2) * sizeof(float);
  return (bytes + 255) & ~size_t(255);
}

static attn_status_t flat_args(const void* q, const void* k, const void* v,
                               const int32_t* kv_indptr, int B, int Hq, int Hkv, int D,
                               int max_kv_len, long long total_kv, float scale, int num_pieces,
                               int dtype, const char* who, rattn::DecodeArgs* a) {
  attn_status_t cs = check_decode(q, k, v, kv_indptr, B, Hq, Hkv, D, max_kv_len, total_kv, scale,
                                  0, dtype);
  if (cs != ATTN_OK) return cs;
  if (dtype == ATTN_F32) return fail(ATTN_EUNSUPPORTED, "%s: 16-bit inputs only", who);
  if (num_pieces < 0 || num_pieces > kMaxPieces)
    return fail(ATTN_EINVAL, "%s: num_pieces %d outside [0, %d]", who, num_pieces, kMaxPieces);
  if (total_kv > 0x7fffffffLL) return fail(ATTN_EUNSUPPORTED, "%s: total_kv above 2^31 - 1", who);
  const int P = num_pieces ? num_pieces : attn_decode_flat_pieces(B, Hq, Hkv, D, total_kv);
  *a = rattn::DecodeArgs{q, k, v, kv_indptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                         B, Hq, Hkv, D, Hq / Hkv, attn_decode_flat_max_splits(max_kv_len, total_kv, P),
                         int(flat_piece_len(total_kv, P)), scale * kLog2e, dtype, 0, 0};
  a->flat = 1;
  a->pieces = P;
  a->total_kv = total_kv;
  return ATTN_OK;
}

attn_status_t attn_decode_splitkv_flat(const void* q, const void* k, const void* v,
                                       const int32_t* kv_indptr, void* o, float* lse, int B,
                                       int Hq, int Hkv, int D, int max_kv_len, long long total_kv,
                                       float scale, int num_pieces, int dtype, void* workspace,
                                       size_t workspace_bytes, void* hip_stream) {
  rattn::DecodeArgs a;
  attn_status_t cs = flat_args(q, k, v, kv_indptr, B, Hq, Hkv, D, max_kv_len, total_kv, scale,
                               num_pieces, dtype, "decode_flat", &a);
  if (cs != ATTN_OK) return cs;
  if (!o) return fail(ATTN_EINVAL, "decode_flat: null output");
  if (!aligned16(o)) return fail(ATTN_EINVAL, "decode_flat: o must be 16-byte aligned");
  const size_t need = attn_decode_flat_workspace_bytes(B, Hq, D, max_kv_len, total_kv, a.pieces);
  if (!workspace || workspace_bytes < need)
    return fail(ATTN_EWORKSPACE, "decode_flat: workspace needs %zu bytes, got %zu", need,
                workspace ? workspace_bytes : size_t(0));
  if (!aligned16(workspace))
    return fail(ATTN_EINVAL, "decode_flat: workspace must be 16-byte aligned");
  const size_t rows = size_t(B) * Hq;
  float* ws = static_cast<float*>(workspace);
  a.o = o;
  a.lse = lse;
  a.o_part = ws;
  a.m_part = ws + size_t(a.s) * rows * D;
  a.l_part = a.m_part + size_t(a.s) * rows;
  return hip_status(rattn::launch_decode_flat(a, static_cast<hipStream_t>(hip_stream)),
                    "decode_flat launch");
}

attn_status_t attn_debug_flat_ranges(const int32_t* kv_indptr, int B, int max_kv_len,
                                     long long total_kv, int num_pieces, int32_t* ranges,
                                     void* hip_stream) {
  if (!kv_indptr || !ranges) return fail(ATTN_EINVAL, "flat_ranges: null pointer");
  if (B < 1 || max_kv_len < 0 || total_kv < 0 || total_kv > 0x7fffffffLL)
    return fail(ATTN_EINVAL, "flat_ranges: bad B, max_kv_len or total_kv");
  if (num_pieces < 1 || num_pieces > kMaxPieces)
    return fail(ATTN_EINVAL, "flat_ranges: num_pieces %d outside [1, %d]", num_pieces, kMaxPieces);
  rattn::DecodeArgs a{};
  a.kv_indptr = kv_indptr;
  a.B = B;
  a.s = attn_decode_flat_max_splits(max_kv_len, total_kv, num_pieces);
  a.chunk = int(flat_piece_len(total_kv, num_pieces));
  a.flat = 1;
  a.pieces = num_pieces;
  a.total_kv = total_kv;
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  hipError_t e = rattn::launch_flat_ranges(a, ranges, st);
  if (e != hipSuccess) return hip_status(e, "flat_ranges launch");
  return hip_status(hipStreamSynchronize(st), "flat_ranges sync");
}

attn_status_t attn_prefill(const void* q, const void* k, const void* v, const int32_t* qo_indptr,
                           const int32_t* kv_indptr, void* o, float* lse, int B, int Hq, int Hkv,
                           int D, int max_q_len, int max_kv_len, float scale, int causal,
                           int dtype, void* hip_stream) {
  if (!q || !k || !v || !qo_indptr || !kv_indptr || !o)
    return fail(ATTN_EINVAL, "prefill: null pointer");
  if (B < 1 || Hq < 1 || Hkv < 1) return fail(ATTN_EINVAL, "prefill: B, Hq, Hkv must be >= 1");
  if (B > 65535 || Hq > 65535) return fail(ATTN_EUNSUPPORTED, "prefill: B or Hq above 65535");
  if ((long long)max_q_len > (long long)rattn::prefill_rows_per_workgroup() * 65535)
    return fail(ATTN_EUNSUPPORTED, "prefill: max_q_len above %lld",
                (long long)rattn::prefill_rows_per_workgroup() * 65535);
  if (Hq % Hkv) return fail(ATTN_EINVAL, "prefill: Hq %d not a multiple of Hkv %d", Hq, Hkv);
  if (D != 64 && D != 128) return fail(ATTN_EUNSUPPORTED, "prefill: D = %d (supported: 64, 128)", D);
  if (dtype != ATTN_BF16 && dtype != ATTN_F16)
    return fail(ATTN_EUNSUPPORTED, "prefill: dtype %d (supported: bf16, f16)", dtype);
  if (max_q_len < 0 || max_kv_len < 0) return fail(ATTN_EINVAL, "prefill: negative length");
  if (causal != 0 && causal != 1) return fail(ATTN_EINVAL, "prefill: causal must be 0 or 1");
  if (!std::isfinite(scale) || !(scale > 0.f))
    return fail(ATTN_EINVAL, "prefill: scale must be finite and positive");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(ATTN_EINVAL, "prefill: q, k, v, o must be 16-byte aligned");
  rattn::PrefillArgs a{q, k, v, qo_indptr, kv_indptr, o, lse, B, Hq, Hkv, D, Hq / Hkv,
                       max_q_len, max_kv_len, scale * kLog2e, causal, dtype,
                       1, 0, nullptr, nullptr, nullptr, 0};
  return hip_status(rattn::launch_prefill(a, static_cast<hipStream_t>(hip_stream)), "prefill launch");
}

size_t attn_prefill_workspace_bytes(long long total_q, int Hq, int D, int num_splits) {
  if (total_q < 0 || Hq < 1 || D < 1 || num_splits < 1) return 0;
  // fp16 partial rows, then fp32 m, l and row scales
  const size_t raw = size_t(num_splits) * size_t(total_q) * size_t(Hq) * (size_t(D) * 2 + 12);
  return (raw + 255) / 256 * 256;
}

int attn_prefill_choose_splits(int B, int Hq, int Hkv, int D, int max_q_len, int max_kv_len) {
  (void)Hkv;
  (void)D;
  if (B <= 0 || Hq <= 0 || max_q_len <= 0 || max_kv_len <= 0) return 1;
  // Two workgroups per compute unit fill the chip; split the keys only when
  // the query tiles alone fall short, and keep chunks of at least 1024 keys.
  const int bq = rattn::prefill_rows_per_workgroup();
  const long long wgs = (long long)B * Hq * ((max_q_len + bq - 1) / bq);
  const long long target = 2LL * attn_device_cu_count();
  if (wgs >= target) return 1;
  long long s = (target + wgs - 1) / wgs;
  const long long s_max = (max_kv_len + 1023) / 1024;
  if (s > s_max) s = s_max;
  if (s > kMaxSplits) s = kMaxSplits;
  return s < 1 ? 1 : int(s);
}

attn_status_t attn_prefill_splitkv(const void* q, const void* k, const void* v,
                                   const int32_t* qo_indptr, const int32_t* kv_indptr, void* o,
                                   float* lse, int B, int Hq, int Hkv, int D, int max_q_len,
                                   int max_kv_len, long long total_q, float scale, int causal,
                                   int num_splits, int dtype, void* workspace,
                                   size_t workspace_bytes, void* hip_stream) {
  if (!q || !k || !v || !qo_indptr || !kv_indptr || !o)
    return fail(ATTN_EINVAL, "prefill_splitkv: null pointer");
  if (B < 1 || Hq < 1 || Hkv < 1) return fail(ATTN_EINVAL, "prefill_splitkv: B, Hq, Hkv must be >= 1");
  if (B > 65535 || Hq > 65535) return fail(ATTN_EUNSUPPORTED, "prefill_splitkv: B or Hq above 65535");
  if (Hq % Hkv) return fail(ATTN_EINVAL, "prefill_splitkv: Hq %d not a multiple of Hkv %d", Hq, Hkv);
  if (D != 64 && D != 128)
    return fail(ATTN_EUNSUPPORTED, "prefill_splitkv: D = %d (supported: 64, 128)", D);
  if (dtype != ATTN_BF16 && dtype != ATTN_F16)
    return fail(ATTN_EUNSUPPORTED, "prefill_splitkv: dtype %d (supported: bf16, f16)", dtype);
  if (max_q_len < 0 || max_kv_len < 0 || total_q < 0)
    return fail(ATTN_EINVAL, "prefill_splitkv: negative length");
  if (causal != 0 && causal != 1) return fail(ATTN_EINVAL, "prefill_splitkv: causal must be 0 or 1");
  if (!std::isfinite(scale) || !(scale > 0.f))
    return fail(ATTN_EINVAL, "prefill_splitkv: scale must be finite and positive");
  if (num_splits < 0 || num_splits > kMaxSplits)
    return fail(ATTN_EINVAL, "prefill_splitkv: num_splits %d outside [0, %d]", num_splits, kMaxSplits);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(ATTN_EINVAL, "prefill_splitkv: q, k, v, o must be 16-byte aligned");
  const int s = num_splits ? num_splits
                           : attn_prefill_choose_splits(B, Hq, Hkv, D, max_q_len, max_kv_len);
  const int bq = rattn::prefill_rows_per_workgroup();
  const long long qtiles = (max_q_len + bq - 1) / bq;
  if (qtiles * s > 65535)
    return fail(ATTN_EUNSUPPORTED, "prefill_splitkv: ceil(max_q_len / %d) * s = %lld above 65535",
                bq, qtiles * s);
  const long long rows = total_q * Hq;
  if (s > 1 && rows > (1LL << 30)) return fail(ATTN_EUNSUPPORTED, "prefill_splitkv: rows above 2^30");
  const size_t need = s > 1 ? attn_prefill_workspace_bytes(total_q, Hq, D, s) : 0;
  if (s > 1 && (!workspace || workspace_bytes < need))
    return fail(ATTN_EWORKSPACE, "prefill_splitkv: workspace needs %zu bytes, got %zu", need,
                workspace ? workspace_bytes : size_t(0));
  if (s > 1 && !aligned16(workspace))
    return fail(ATTN_EINVAL, "prefill_splitkv: workspace must be 16-byte aligned");
  const int chunk = max_kv_len > 0 ? (max_kv_len + s - 1) / s : 0;
  // workspace: fp16 o_part [s, rows, D], then fp32 m_part, l_part, x_part [s, rows]
  uint16_t* wo = static_cast<uint16_t*>(workspace);
  float* wf = reinterpret_cast<float*>(wo + size_t(s) * size_t(rows) * D);
  rattn::PrefillArgs a{q, k, v, qo_indptr, kv_indptr, o, lse, B, Hq, Hkv, D, Hq / Hkv,
                       max_q_len, max_kv_len, scale * kLog2e, causal, dtype,
                       s, chunk,
                       s > 1 ? wo : nullptr,
                       s > 1 ? wf : nullptr,
                       s > 1 ? wf + size_t(s) * size_t(rows) : nullptr,
                       rows,
                       s > 1 ? wf + 2 * size_t(s) * size_t(rows) : nullptr};
  return hip_status(rattn::launch_prefill(a, static_cast<hipStream_t>(hip_stream)),
                    "prefill_splitkv launch");
}

// One L x L mask into the two-level format, appended after f_base full and
// p_base part tiles already written: indptr entries qb = 0 .. nb (values
// global, i.e. offset by the bases), kblock / bits entries from the bases
// on.  fill = false only counts.
static attn_status_t encode_mask(const uint8_t* dense, int L, int f_base, int p_base,
                                 int32_t* full_indptr, int32_t* full_kblock, int32_t* part_indptr,
                                 int32_t* part_kblock, uint64_t* part_bits, bool fill, int f_cap,
                                 int p_cap, int* nf_out, int* np_out) {
  const int nb = L / 64;
  int nf = f_base, np = p_base;
  if (fill) {
    full_indptr[0] = nf;
    part_indptr[0] = np;
  }
  for (int qb = 0; qb < nb; ++qb) {
    for (int kb = 0; kb < nb; ++kb) {
      uint64_t words[64];
      int valid = 0;
      for (int ir = 0; ir < 8; ++ir)
        for (int ic = 0; ic < 8; ++ic) {
          uint64_t wd = 0;
          for (int r = 0; r < 8; ++r)
            for (int c = 0; c < 8; ++c) {
              const size_t row = size_t(qb) * 64 + ir * 8 + r;
              const size_t col = size_t(kb) * 64 + ic * 8 + c;
              if (dense[row * size_t(L) + col]) {
                wd |= uint64_t(1) << (r * 8 + c);
                ++valid;
              }
            }
          words[ir * 8 + ic] = wd;
        }
      if (valid == 0) continue;  // empty OT: not stored
      if (valid == 64 * 64) {
        if (fill) {
          if (nf >= f_cap) return fail(ATTN_EINVAL, "bsr_encode: nnz_full too small");
          full_kblock[nf] = kb;
        }
        ++nf;
      } else {
        if (fill) {
          if (np >= p_cap) return fail(ATTN_EINVAL, "bsr_encode: nnz_part too small");
          part_kblock[np] = kb;
          std::memcpy(part_bits + size_t(np) * 64, words, sizeof words);
        }
        ++np;
      }
    }
    if (fill) {
      full_indptr[qb + 1] = nf;
      part_indptr[qb + 1] = np;
    }
  }
  *nf_out = nf;
  *np_out = np;
  return ATTN_OK;
}

attn_status_t attn_bsr_encode_host_stacked(const uint8_t* dense, int num_masks, int L,
                                           int32_t* full_indptr, int32_t* full_kblock,
                                           int32_t* part_indptr, int32_t* part_kblock,
                                           uint64_t* part_bits, int* nnz_full, int* nnz_part) {
  if (!dense || !nnz_full || !nnz_part) return fail(ATTN_EINVAL, "bsr_encode: null pointer");
  if (L <= 0 || L % 64) return fail(ATTN_EINVAL, "bsr_encode: L = %d is not a positive multiple of 64", L);
  if (num_masks < 1) return fail(ATTN_EINVAL, "bsr_encode: num_masks %d < 1", num_masks);
  const bool fill = full_indptr || full_kblock || part_indptr || part_kblock || part_bits;
  if (fill && !(full_indptr && part_indptr && part_bits && (full_kblock || *nnz_full == 0) &&
                (part_kblock || *nnz_part == 0)))
    return fail(ATTN_EINVAL, "bsr_encode: fill pass needs every output array");
  const int nb = L / 64;
  int nf = 0, np = 0;
  for (int m = 0; m < num_masks; ++m) {
    const uint8_t* dm = dense + size_t(m) * size_t(L) * size_t(L);
    attn_status_t st = encode_mask(dm, L, nf, np, fill ? full_indptr + size_t(m) * (nb + 1) : nullptr,
                                   full_kblock, fill ? part_indptr + size_t(m) * (nb + 1) : nullptr,
                                   part_kblock, part_bits, fill, *nnz_full, *nnz_part, &nf, &np);
    if (st != ATTN_OK) return st;
  }
  if (fill && (nf != *nnz_full || np != *nnz_part))
    return fail(ATTN_EINVAL, "bsr_encode: sizes differ from the mask (%d/%d full, %d/%d part)", nf,
                *nnz_full, np, *nnz_part);
  *nnz_full = nf;
  *nnz_part = np;
  return ok();
}

attn_status_t attn_bsr_encode_host(const uint8_t* dense, int L, int32_t* full_indptr,
                                   int32_t* full_kblock, int32_t* part_indptr,
                                   int32_t* part_kblock, uint64_t* part_bits, int* nnz_full,
                                   int* nnz_part) {
  return attn_bsr_encode_host_stacked(dense, 1, L, full_indptr, full_kblock, part_indptr,
                                      part_kblock, part_bits, nnz_full, nnz_part);
}

static attn_status_t check_mask(const attn_bsr_mask* m, const char* who) {
  if (!m) return fail(ATTN_EINVAL, "%s: null mask", who);
  if (m->seq_len <= 0 || m->seq_len % 64)
    return fail(ATTN_EINVAL, "%s: mask seq_len %d not a positive multiple of 64", who, m->seq_len);
  if (m->num_blocks != m->seq_len / 64)
    return fail(ATTN_EINVAL, "%s: mask num_blocks %d != seq_len / 64", who, m->num_blocks);
  if (m->nnz_full < 0 || m->nnz_part < 0) return fail(ATTN_EINVAL, "%s: negative nnz", who);
  if (!m->full_indptr || !m->part_indptr) return fail(ATTN_EINVAL, "%s: null mask indptr", who);
  if ((m->nnz_full && !m->full_kblock) || (m->nnz_part && (!m->part_kblock || !m->part_bits)))
    return fail(ATTN_EINVAL, "%s: null mask array", who);
  return ATTN_OK;
}

// Shared validation of the block-sparse prefill entry points; fills a.
static attn_status_t bsr_args(const void* q, const void* k, const void* v,
                              const attn_bsr_mask* mask, int num_masks, void* o, float* lse, int B,
                              int L, int Hq, int Hkv, int D, float scale, int dtype,
                              rattn::BsrArgs* a) {
  if (!q || !k || !v || !o) return fail(ATTN_EINVAL, "prefill_bsr: null pointer");
  attn_status_t ms = check_mask(mask, "prefill_bsr");
  if (ms != ATTN_OK) return ms;
  if (B < 1 || Hq < 1 || Hkv < 1) return fail(ATTN_EINVAL, "prefill_bsr: B, Hq, Hkv must be >= 1");
  if (B > 65535 || Hq > 65535) return fail(ATTN_EUNSUPPORTED, "prefill_bsr: B or Hq above 65535");
  if (L != mask->seq_len) return fail(ATTN_EINVAL, "prefill_bsr: L %d != mask seq_len %d", L, mask->seq_len);
  if (Hq % Hkv) return fail(ATTN_EINVAL, "prefill_bsr: Hq %d not a multiple of Hkv %d", Hq, Hkv);
  if (num_masks < 1 || Hq % num_masks)
    return fail(ATTN_EINVAL, "prefill_bsr: num_masks %d does not divide Hq %d", num_masks, Hq);
  if (D != 64 && D != 128) return fail(ATTN_EUNSUPPORTED, "prefill_bsr: D = %d (supported: 64, 128)", D);
  if (dtype != ATTN_BF16 && dtype != ATTN_F16)
    return fail(ATTN_EUNSUPPORTED, "prefill_bsr: dtype %d (supported: f16, bf16)", dtype);
  if (!std::isfinite(scale) || !(scale > 0.f))
    return fail(ATTN_EINVAL, "prefill_bsr: scale must be finite and positive");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(ATTN_EINVAL, "prefill_bsr: q, k, v, o must be 16-byte aligned");
  if (mask->nnz_part && (reinterpret_cast<uintptr_t>(mask->part_bits) & 7u))
    return fail(ATTN_EINVAL, "prefill_bsr: part_bits must be 8-byte aligned");
  *a = rattn::BsrArgs{q, k, v, mask->full_indptr, mask->full_kblock, mask->part_indptr,
                      mask->part_kblock, mask->part_bits, o, lse, B, L, Hq, Hkv, D, Hq / Hkv,
                      mask->num_blocks, scale * kLog2e, dtype, Hq / num_masks};
  return ATTN_OK;
}

attn_status_t attn_prefill_bsr_heads(const void* q, const void* k, const void* v,
                                     const attn_bsr_mask* mask, int num_masks, void* o, float* lse,
                                     int B, int L, int Hq, int Hkv, int D, float scale, int dtype,
                                     void* hip_stream) {
  rattn::BsrArgs a;
  attn_status_t st = bsr_args(q, k, v, mask, num_masks, o, lse, B, L, Hq, Hkv, D, scale, dtype, &a);
  if (st != ATTN_OK) return st;
  return hip_status(rattn::launch_prefill_bsr(a, static_cast<hipStream_t>(hip_stream)),
                    "prefill_bsr launch");
}

attn_status_t attn_prefill_bsr_rows(const void* q, const void* k, const void* v,
                                    const attn_bsr_mask* mask, int num_masks, void* o, float* lse,
                                    int B, int L, int Hq, int Hkv, int D, float scale, int dtype,
                                    void* hip_stream) {
  rattn::BsrArgs a;
  attn_status_t st = bsr_args(q, k, v, mask, num_masks, o, lse, B, L, Hq, Hkv, D, scale, dtype, &a);
  if (st != ATTN_OK) return st;
  return hip_status(rattn::launch_prefill_bsr_rows(a, static_cast<hipStream_t>(hip_stream)),
                    "prefill_bsr_rows launch");
}

// Modelled time of the two block-sparse kernels on MI355X, in us: a launch
// floor plus a cost per unit of work summed over heads and batch entries
// (per stored outer tile for the block-wise kernel, per (16-row slab,
// 16-key block) for the row-wise one).  Fitted (least squares on relative
// error) to kernel-trace durations of both kernels over nine mask families
// at L 1024 and 4096, D 64 and 128 (fp16, 16 heads): the model picks the
// faster kernel in 34 of the 36 cases; the two others are ties within
// 0.7 us.
struct BsrCost { double b0, b1, r0, r1; };
static BsrCost bsr_cost(int D) {
  return D == 64 ? BsrCost{7.2, 1.68e-3, 7.1, 0.336e-3} : BsrCost{9.9, 4.36e-3, 6.8, 0.671e-3};
}

attn_status_t attn_bsr_plan_host(const int32_t* full_indptr, const int32_t* part_indptr,
                                 const uint64_t* part_bits, int num_masks, int L, int Hq, int B,
                                 int D, attn_bsr_plan* plan) {
  if (!full_indptr || !part_indptr || !plan) return fail(ATTN_EINVAL, "bsr_plan: null pointer");
  if (L <= 0 || L % 64) return fail(ATTN_EINVAL, "bsr_plan: L = %d is not a positive multiple of 64", L);
  if (num_masks < 1 || Hq < 1 || B < 1 || Hq % num_masks)
    return fail(ATTN_EINVAL, "bsr_plan: need num_masks >= 1 dividing Hq >= 1, B >= 1");
  if (D != 64 && D != 128) return fail(ATTN_EUNSUPPORTED, "bsr_plan: D = %d (supported: 64, 128)", D);
  const int nb = L / 64;
  long long ots = 0, units = 0;
  for (int m = 0; m < num_masks; ++m) {
    const int32_t* fi = full_indptr + size_t(m) * (nb + 1);
    const int32_t* pi = part_indptr + size_t(m) * (nb + 1);
    for (int qb = 0; qb < nb; ++qb) {
      const long long nf = fi[qb + 1] - fi[qb], np = pi[qb + 1] - pi[qb];
      if (nf < 0 || np < 0) return fail(ATTN_EINVAL, "bsr_plan: indptr not monotone");
      if (np && !part_bits) return fail(ATTN_EINVAL, "bsr_plan: null part_bits");
      ots += nf + np;
      units += 16 * nf;  // a full tile: 4 slabs x 4 key blocks
      for (int p = pi[qb]; p < pi[qb + 1]; ++p) {
        const uint64_t* wd = part_bits + size_t(p) * 64;
        for (int slab = 0; slab < 4; ++slab)
          for (int kb = 0; kb < 4; ++kb) {
            const int r0 = 2 * slab * 8, r1 = (2 * slab + 1) * 8;
            if (wd[r0 + 2 * kb] | wd[r0 + 2 * kb + 1] | wd[r1 + 2 * kb] | wd[r1 + 2 * kb + 1]) ++units;
          }
      }
    }
  }
  // each mask serves Hq / num_masks heads of every batch entry
  const double reps = double(Hq / num_masks) * B;
  const BsrCost c = bsr_cost(D);
  plan->stored_ots = ots;
  plan->row_blocks = units;
  plan->block_cost = c.b0 + c.b1 * double(ots) * reps;
  plan->row_cost = c.r0 + c.r1 * double(units) * reps;
  plan->kernel = plan->row_cost < plan->block_cost ? ATTN_BSR_ROWWISE : ATTN_BSR_BLOCKWISE;
  return ok();
}

attn_status_t attn_prefill_bsr(const void* q, const void* k, const void* v,
                               const attn_bsr_mask* mask, void* o, float* lse, int B, int L, int Hq,
                               int Hkv, int D, float scale, int dtype, void* hip_stream) {
  return attn_prefill_bsr_heads(q, k, v, mask, 1, o, lse, B, L, Hq, Hkv, D, scale, dtype,
                                hip_stream);
}

attn_status_t attn_debug_split_ranges(const int32_t* kv_indptr, int B, int max_kv_len,
                                      int num_splits, int32_t* ranges, void* hip_stream) {
  if (!kv_indptr || !ranges) return fail(ATTN_EINVAL, "split_ranges: null pointer");
  if (B < 1 || max_kv_len < 0) return fail(ATTN_EINVAL, "split_ranges: bad B or max_kv_len");
  if (num_splits < 1 || num_splits > kMaxSplits)
    return fail(ATTN_EINVAL, "split_ranges: num_splits %d outside [1, %d]", num_splits, kMaxSplits);
  const int chunk = max_kv_len > 0 ? (max_kv_len + num_splits - 1) / num_splits : 0;
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  hipError_t e = rattn::launch_split_ranges(kv_indptr, B, num_splits, chunk, ranges, st);
  if (e != hipSuccess) return hip_status(e, "split_ranges launch");
  return hip_status(hipStreamSynchronize(st), "split_ranges sync");
}

attn_status_t attn_debug_bsr_decode(const attn_bsr_mask* mask, uint8_t* dense, void* hip_stream) {
  attn_status_t ms = check_mask(mask, "bsr_decode");
  if (ms != ATTN_OK) return ms;
  if (!dense) return fail(ATTN_EINVAL, "bsr_decode: null output");
  if (mask->nnz_part && (reinterpret_cast<uintptr_t>(mask->part_bits) & 7u))
    return fail(ATTN_EINVAL, "bsr_decode: part_bits must be 8-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  hipError_t e = rattn::launch_bsr_decode(mask->full_indptr, mask->full_kblock, mask->part_indptr,
                                          mask->part_kblock, mask->part_bits, mask->num_blocks,
                                          dense, st);
  if (e != hipSuccess) return hip_status(e, "bsr_decode launch");
  return hip_status(hipStreamSynchronize(st), "bsr_decode sync");
}

}  // extern "C"
