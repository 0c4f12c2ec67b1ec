// attn_core.hpp -- the fused attention tile step shared by the dense/causal
// prefill kernel and the block-sparse kernel (gfx950, 32x32x16 MFMA).
//
// One wave owns 32 query rows.  Keys arrive in tiles of BK (32 or 64)
// staged in LDS (iterative tiling of the key dimension, Cleave article on
// tip.co.jp, "複数リダクションのスケジューリング"); for each tile the wave
// computes the transposed score block S^T = K Q^T, updates the row max and
// the row sum of exp over that same block in one pass (horizontal fusion),
// rescales its output accumulator when the max moved, and adds V^T P^T.
// Working on S^T puts one query per lane column, so each row's max and sum
// are lane-local plus a single exchange with the partner lane l ^ 32.
//
// LDS layout per stage:
//   K tile  [BK keys][D + 8] (natural row order; +16 B pad per row spreads
//           the 32 rows one MFMA operand read touches over all banks)
//   V^T tile [D][BK + 8] with keys stored in "slot order":
//           key k = 16*T + 8*a + 4*h + b  ->  position 16*T + 8*h + 4*a + b,
//           so that the eight reduction slots lane half h feeds to one
//           V^T P^T MFMA are 16 contiguous bytes.
#pragma once
#include "device.hpp"

namespace rattn {

template <int D, int BK_>
struct TileGeom {
  static constexpr int BK = BK_;          // keys per tile (32 or 64)
  static constexpr int NKB = BK / 32;     // 32-key score blocks per tile
  static constexpr int KLD = D + 8;       // K row stride (elements)
  static constexpr int VLD = BK + 8;      // V^T row stride (elements)
  static constexpr int K_ELEMS = BK * KLD;
  static constexpr int V_ELEMS = D * VLD;
  static constexpr int STAGE = K_ELEMS + V_ELEMS;  // 16-bit elements per stage
};

// Registers carrying one K/V tile from global memory to its LDS stage.  The
// workgroup's NT threads split by role: threads [0, NT/2) carry V in items
// of 4 keys x 8 dims (stored transposed), threads [NT/2, NT) carry K in
// 16-byte chunks; both roles issue about the same number of loads.
template <int D, int BK, int NT>
struct TileRegs {
  static constexpr int HALF = NT / 2;
  static constexpr int KCHUNKS = BK * (D / 8);        // 16-byte K chunks per tile
  static constexpr int VITEMS = (BK / 4) * (D / 8);   // 4-key x 8-dim V items per tile
  static constexpr int KPT = (KCHUNKS + HALF - 1) / HALF;
  static constexpr int VPT = (VITEMS + HALF - 1) / HALF;
  static constexpr int N = KPT > 4 * VPT ? KPT : 4 * VPT;
  u32x4 r[N];
};

// The role of a thread's wave (K or V carrier), as a wave-uniform scalar so
// the role split costs a scalar branch rather than exec-mask juggling.
template <int NT>
__device__ __forceinline__ bool k_role(int tid) {
  return __builtin_amdgcn_readfirstlane(tid) >= NT / 2;
}

// Global -> registers: K rows kkey0 .. kkey0+BK-1 (if do_k) and V rows
// vkey0 .. vkey0+BK-1 (if do_v) of a request of n_keys keys; the two may
// belong to different tiles.  Each role reads through a buffer resource that
// ends at the request's last key, so rows past it come back as zeros without
// a memory access (their scores are masked, and a zero V row adds nothing).
// A thread's offsets into the tile are fixed, so a tile costs a few scalar
// instructions for the resource and no per-load address arithmetic.
template <int D, int BK, int NT>
__device__ __forceinline__ void tile_load(TileRegs<D, BK, NT>& rr, const uint16_t* kbase,
                                          const uint16_t* vbase, int row_stride, int kkey0,
                                          int vkey0, int n_keys, int tid, bool do_k = true,
                                          bool do_v = true) {
  typedef TileRegs<D, BK, NT> R;
  constexpr int CPR = D / 8, HALF = NT / 2;
  static_assert(HALF % CPR == 0 && HALF % (BK / 4) == 0, "role split must tile the rows");
  if (k_role<NT>(tid)) {
    if (!do_k) return;
    const __amdgpu_buffer_rsrc_t rs =
        buffer_rsrc(kbase + int64_t(kkey0) * row_stride, int64_t(n_keys - kkey0) * row_stride * 2);
    // chunk t + HALF*x: row t/CPR + x*HALF/CPR, dims 8*(t%CPR) ..
    const int t = tid - HALF;
    const int base = ((t / CPR) * row_stride + 8 * (t % CPR)) * 2;
#pragma unroll
    for (int x = 0; x < R::KPT; ++x)
      if (R::KPT * HALF == R::KCHUNKS || t + HALF * x < R::KCHUNKS)
        rr.r[x] = buffer_load128(rs, base + x * (HALF / CPR) * row_stride * 2);
  } else {
    if (!do_v) return;
    const __amdgpu_buffer_rsrc_t rs =
        buffer_rsrc(vbase + int64_t(vkey0) * row_stride, int64_t(n_keys - vkey0) * row_stride * 2);
    // item tid + HALF*x: keys 4*(tid % (BK/4)) .. +4, dims 8*(tid/(BK/4) + x*HALF/(BK/4)) ..
    const int base = (4 * (tid % (BK / 4)) * row_stride + 8 * (tid / (BK / 4))) * 2;
#pragma unroll
    for (int x = 0; x < R::VPT; ++x)
      if (R::VPT * HALF == R::VITEMS || tid + HALF * x < R::VITEMS) {
#pragma unroll
        for (int b = 0; b < 4; ++b)
          rr.r[4 * x + b] = buffer_load128(rs, base + (b * row_stride + 8 * x * (HALF / (BK / 4))) * 2);
      }
  }
}

// Registers -> LDS: the K tile, natural, at kdst (if do_k); the V tile,
// transposed into slot order, at vdst (if do_v).
template <int D, int BK, int NT>
__device__ __forceinline__ void tile_store(const TileRegs<D, BK, NT>& rr, uint16_t* kdst,
                                           uint16_t* vdst, int tid, bool do_k = true,
                                           bool do_v = true) {
  typedef TileGeom<D, BK> Gm;
  typedef TileRegs<D, BK, NT> R;
  constexpr int CPR = D / 8, HALF = NT / 2;
  if (k_role<NT>(tid)) {
    if (!do_k) return;
    // chunk t + HALF*x goes to row t/CPR + x*HALF/CPR: one base register,
    // the rest immediate offsets
    const int t = tid - HALF;
    uint16_t* kp = kdst + (t / CPR) * Gm::KLD + 8 * (t % CPR);
#pragma unroll
    for (int x = 0; x < R::KPT; ++x)
      if (R::KPT * HALF == R::KCHUNKS || t + HALF * x < R::KCHUNKS)
        *reinterpret_cast<u32x4*>(kp + x * (HALF / CPR) * Gm::KLD) = rr.r[x];
  } else {
    if (!do_v) return;
    // item tid + HALF*x: keys 4*kg .. 4*kg+3 with kg = tid % (BK/4) (so
    // T = kg / 4, a = (kg / 2) % 2, h = kg % 2), dims 8*dc .. with
    // dc = tid / (BK/4) + x*HALF/(BK/4)
    const int kg = tid % (BK / 4);
    const int pos = 16 * (kg >> 2) + 8 * (kg & 1) + 4 * ((kg >> 1) & 1);
    uint16_t* vp = vdst + 8 * (tid / (BK / 4)) * Gm::VLD + pos;
#pragma unroll
    for (int x = 0; x < R::VPT; ++x)
      if (R::VPT * HALF == R::VITEMS || tid + HALF * x < R::VITEMS) {
        const u32x4* v = rr.r + 4 * x;
#pragma unroll
        for (int jd = 0; jd < 8; ++jd) {
          const int w = jd >> 1;
          u32x2 pk;
          if (jd & 1) {
            pk[0] = pack_hi(v[0][w], v[1][w]);
            pk[1] = pack_hi(v[2][w], v[3][w]);
          } else {
            pk[0] = pack_lo(v[0][w], v[1][w]);
            pk[1] = pack_lo(v[2][w], v[3][w]);
          }
          *reinterpret_cast<u32x2*>(vp + (8 * x * (HALF / (BK / 4)) + jd) * Gm::VLD) = pk;
        }
      }
  }
}

// Per-wave running state of 32 query rows (one per lane column).
template <int D>
struct RowState {
  f32x16 o[D / 32];  // O^T accumulators: o[db][r] is dim 32*db + 8*(r/4) + 4*h + r%4
  float m;           // running reference max (log2 units), equal in lanes l and l^32
  float l;           // this lane's share of the running sum
};

template <int D>
__device__ __forceinline__ void row_state_init(RowState<D>& st) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) st.o[db][r] = 0.f;
  st.m = -INFINITY;
  st.l = 0.f;
}

// Q^T operand of the wave's 32 rows: slab u, lane half h -> dims 16u + 8h .. +8.
// The empty asm statements consume the loaded registers right away, so the
// loads are complete on every path into the tile loop.  Otherwise the
// compiler, unsure whether they are still in flight inside the loop, puts a
// wait on them before each score MFMA, and since loads complete in order
// that wait also drains the prefetch of later tiles.
template <int D>
__device__ __forceinline__ void load_q(u32x4 (&qb)[D / 16], const uint16_t* qrow, int lane) {
  const int h = lane >> 5;
#pragma unroll
  for (int u = 0; u < D / 16; ++u) qb[u] = ldg128(qrow + 16 * u + 8 * h);
#pragma unroll
  for (int u = 0; u < D / 16; ++u) __asm__ volatile("" ::"v"(qb[u]));
}

// One 32-key block of S^T: s[r] = q(lane%32) . k(32*kb + 8*(r/4) + 4*h + r%4)
// over the K tile at klds.
template <class T, int D, int BK>
__device__ __forceinline__ void qk_block(f32x16& s, const uint16_t* klds, int kb,
                                         const u32x4 (&qb)[D / 16], int lane) {
  typedef typename T::vec8 vec8;
  typedef TileGeom<D, BK> Gm;
  const uint16_t* kp = klds + (32 * kb + (lane & 31)) * Gm::KLD + 8 * (lane >> 5);
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
  for (int u = 0; u < D / 16; ++u) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(kp + 16 * u);
    acc = T::mfma32(as<vec8>(a), as<vec8>(qb[u]), acc);
  }
  s = acc;
}

// S^T for one tile: s[kb] for every 32-key block.
template <class T, int D, int BK>
__device__ __forceinline__ void qk_tile(f32x16 (&s)[BK / 32], const uint16_t* klds,
                                        const u32x4 (&qb)[D / 16], int lane) {
#pragma unroll
  for (int kb = 0; kb < BK / 32; ++kb) qk_block<T, D, BK>(s[kb], klds, kb, qb, lane);
}

// The running reference max m of a row is raised only when a tile's max
// exceeds it by more than this many log2 units; until then the tile's
// weights exp2(score - m) may reach 2^kRescaleSlack.  The result is the same
// (every weight and the sum share the same reference), but most tiles skip
// the rescale of the output accumulator.
constexpr float kRescaleSlack = 8.f;

// Online softmax, step 1: the tile's row max over raw scores (masked
// entries -inf), the same in lanes l and l ^ 32.
template <int NKB>
__device__ __forceinline__ float tile_rowmax(const f32x16 (&s)[NKB], int xaddr) {
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; r += 2) mx = max3(mx, s[kb][r], s[kb][r + 1]);
  (void)xaddr;
  return max_halves(mx);
}

// Step 2: raise the reference max to the tile max mx (raw score units; c =
// scale * log2(e) turns a score into log2 units) when it exceeds the
// reference by more than the slack, rescaling O and l.  The branch is taken
// by few tiles and is uniform over the wave.
template <int D>
__device__ __forceinline__ void raise_ref(RowState<D>& st, float mx, float c) {
  const float mxs = mx * c;
  const bool need = mxs > st.m + kRescaleSlack;  // st.m = -inf: any valid key
  if (__any(need)) {
    const float m_new = need ? mxs : st.m;
    const float alpha = need ? fexp2(st.m - m_new) : 1.f;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) st.o[db] *= alpha;
    st.l *= alpha;
    st.m = m_new;
  }
}

// The reference the weights are taken against; st.m = -inf means no valid
// key so far, where every score is -inf and every weight 0.
template <int D>
__device__ __forceinline__ float ref_max(const RowState<D>& st) {
  return st.m == -INFINITY ? 0.f : st.m;
}

// Step 3, one 32-key block: weights exp2(s*c - mref), added to l and returned
// as the bf16/f16 operands pb of the value update.  (The sum is taken before
// the rounding to 16 bits: a row with few keys would otherwise carry up to
// 2^-9 relative error in its sum.)
template <class T>
__device__ __forceinline__ void exp_block(float& l, const f32x16& s, float c, float mref,
                                          typename T::vec8 (&pb)[2]) {
  float psum = 0.f;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    f32x8 p;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      p[i] = fexp2(__builtin_fmaf(s[8 * t + i], c, -mref));
      psum += p[i];
    }
    pb[t] = T::cvt8(p);
  }
  l += psum;
}

// Steps 1 and 2 for a whole tile; returns the reference of its weights.
template <int D, int NKB>
__device__ __forceinline__ float softmax_max(RowState<D>& st, const f32x16 (&s)[NKB], float c,
                                             int xaddr) {
  raise_ref<D>(st, tile_rowmax<NKB>(s, xaddr), c);
  return ref_max<D>(st);
}

// Step 3 for a whole tile.
template <class T, int D, int NKB>
__device__ __forceinline__ void softmax_exp(RowState<D>& st, const f32x16 (&s)[NKB], float c,
                                            float mref, typename T::vec8 (&pb)[NKB][2]) {
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) exp_block<T>(st.l, s[kb], c, mref, pb[kb]);
}

// O^T += V^T P^T over the LDS V^T tile.
template <class T, int D, int BK>
__device__ __forceinline__ void pv_tile(RowState<D>& st, const typename T::vec8 (&pb)[BK / 32][2],
                                        const uint16_t* vlds, int lane) {
  typedef typename T::vec8 vec8;
  typedef TileGeom<D, BK> Gm;
  const uint16_t* vp = vlds + (lane & 31) * Gm::VLD + 8 * (lane >> 5);
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int kb = 0; kb < Gm::NKB; ++kb)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(vp + 32 * db * Gm::VLD + 32 * kb + 16 * t);
        st.o[db] = T::mfma32(as<vec8>(a), pb[kb][t], st.o[db]);
      }
}

// Multi-block forms for a wave that owns RB blocks of 32 query rows: every
// K or V operand read from LDS feeds RB MFMAs, one per row block.
template <class T, int D, int BK, int RB>
__device__ __forceinline__ void qk_tile_rb(f32x16 (&s)[RB][BK / 32], const uint16_t* lds,
                                           const u32x4 (&qb)[RB][D / 16], int lane) {
  typedef typename T::vec8 vec8;
  typedef TileGeom<D, BK> Gm;
  const int row = lane & 31, h = lane >> 5;
#pragma unroll
  for (int kb = 0; kb < Gm::NKB; ++kb) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[rb][kb][r] = 0.f;
    const uint16_t* kp = lds + (32 * kb + row) * Gm::KLD + 8 * h;
#pragma unroll
    for (int u = 0; u < D / 16; ++u) {
      const u32x4 a = *reinterpret_cast<const u32x4*>(kp + 16 * u);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        s[rb][kb] = T::mfma32(as<vec8>(a), as<vec8>(qb[rb][u]), s[rb][kb]);
    }
  }
}

template <class T, int D, int BK, int RB>
__device__ __forceinline__ void pv_tile_rb(RowState<D> (&st)[RB],
                                           const typename T::vec8 (&pb)[RB][BK / 32][2],
                                           const uint16_t* vlds, int lane) {
  typedef typename T::vec8 vec8;
  typedef TileGeom<D, BK> Gm;
  const uint16_t* vp = vlds + (lane & 31) * Gm::VLD + 8 * (lane >> 5);
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int kb = 0; kb < Gm::NKB; ++kb)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(vp + 32 * db * Gm::VLD + 32 * kb + 16 * t);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          st[rb].o[db] = T::mfma32(as<vec8>(a), pb[rb][kb][t], st[rb].o[db]);
      }
}

template <class T, int D, int BK>
__device__ __forceinline__ void softmax_pv(RowState<D>& st, const f32x16 (&s)[BK / 32], float c,
                                           const uint16_t* vlds, int lane) {
  typename T::vec8 pb[BK / 32][2];
  const float mref = softmax_max<D, BK / 32>(st, s, c, (lane ^ 32) << 2);
  softmax_exp<T, D, BK / 32>(st, s, c, mref, pb);
  pv_tile<T, D, BK>(st, pb, vlds, lane);
}

// Final normalisation and store of the wave's 32 rows, through LDS: the
// accumulator layout gives each lane 4 dims of its row per register group,
// so a direct store instruction would write 16 bytes into each of 32 rows.
// Here the rows go to `stage` (the wave's own LDS area of 32 * (2D + 16)
// bytes, free by then) and come back as 16-byte row pieces: each store
// instruction writes 64 / (D / 8) whole rows.  obase points at dim 0 of the
// wave's first row, rows ostride elements apart; rows nvalid .. 31 are not
// written.  lse_out points at the LSE slot of this lane's row (lane % 32),
// or is nullptr.
template <class T, int D>
__device__ __forceinline__ void row_store_staged(const RowState<D>& st, uint16_t* obase, int64_t ostride,
                                                 int nvalid, float* lse_out,
                                                 __attribute__((address_space(3))) char* stage, int lane) {
  constexpr int RS = 2 * D + 16;        // LDS bytes per row
  constexpr int LPR = 2 * D / 16;       // lanes per row on the way out
  constexpr int RPI = 64 / LPR;         // rows per store instruction
  float l = sum_halves(st.l);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const int h = lane >> 5, l32 = lane & 31;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      f32x8 y;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        y[e] = st.o[db][4 * g4 + e] * inv;
        y[4 + e] = 0.f;
      }
      const u32x4 bits = __builtin_bit_cast(u32x4, T::cvt8(y));
      *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(stage + l32 * RS + 2 * (32 * db + 8 * g4 + 4 * h)) =
          u32x2{bits[0], bits[1]};
    }
  // one wave's LDS accesses complete in issue order; the fences keep the
  // compiler from moving the reads above the writes
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int rr = lane / LPR, cc = lane % LPR;
#pragma unroll
  for (int k = 0; k < 32 / RPI; ++k) {
    const int r = RPI * k + rr;
    const u32x4 v = *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(stage + r * RS + 16 * cc);
    if (r < nvalid) *reinterpret_cast<u32x4*>(obase + r * ostride + 8 * cc) = v;
  }
  if (lse_out && h == 0) *lse_out = l > 0.f ? (st.m + flog2(l)) * kLn2 : -INFINITY;
}

// A split's partial result for the wave's 32 rows: O normalised by the
// split's own sum and divided by a power of two 2^e per row (e the binary
// exponent of the row's largest magnitude, so every stored value lies in
// [-1, 1], where fp16 keeps 11 significant bits: a stored element is off by
// at most 2^-12 of the row's largest value, and neither the inputs' range
// nor fp16's can overflow it), the scale 2^e, the reference max m in
// natural-log units and the sum l relative to it; a row without valid keys
// gets O = 0, scale 1, m = -inf, l = 0.  The rows go out through the
// wave's LDS area `stage` (32 * (2D + 16) bytes, free by then) as 16-byte
// row pieces, as in row_store_staged.  obase points at dim 0 of the wave's
// first row in the partial output, rows ostride elements apart; rows
// nvalid .. 31 are not written.  m_out, l_out and x_out point at this
// lane's row (lane % 32), or are nullptr when it does not exist.
template <int D>
__device__ __forceinline__ void row_store_partial_staged(const RowState<D>& st, uint16_t* obase,
                                                         int64_t ostride, int nvalid, float* m_out,
                                                         float* l_out, float* x_out,
                                                         __attribute__((address_space(3))) char* stage,
                                                         int lane) {
  constexpr int RS = 2 * D + 16;        // LDS bytes per row
  constexpr int LPR = 2 * D / 16;       // lanes per row on the way out
  constexpr int RPI = 64 / LPR;         // rows per store instruction
  const float l = sum_halves(st.l);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  float amax = 0.f;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) amax = fmaxf(amax, fabsf(st.o[db][r]));
  int e = __builtin_amdgcn_frexp_expf(max_halves(amax) * inv);
  e = e < -126 ? -126 : (e > 127 ? 127 : e);
  const int h = lane >> 5, l32 = lane & 31;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      f32x8 y;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        y[k] = __builtin_amdgcn_ldexpf(st.o[db][4 * g4 + k] * inv, -e);
        y[4 + k] = 0.f;
      }
      const u32x4 bits = __builtin_bit_cast(u32x4, F16::cvt8(y));
      *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(stage + l32 * RS + 2 * (32 * db + 8 * g4 + 4 * h)) =
          u32x2{bits[0], bits[1]};
    }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int rr = lane / LPR, cc = lane % LPR;
#pragma unroll
  for (int k = 0; k < 32 / RPI; ++k) {
    const int r = RPI * k + rr;
    const u32x4 v = *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(stage + r * RS + 16 * cc);
    if (r < nvalid) *reinterpret_cast<u32x4*>(obase + r * ostride + 8 * cc) = v;
  }
  if (m_out && h == 0) {
    *m_out = l > 0.f ? st.m * kLn2 : -INFINITY;
    *l_out = l;
    *x_out = __builtin_amdgcn_ldexpf(1.f, e);
  }
}

// ---------------------------------------------------------------------------
// Natural-layout tiles written straight from global memory into LDS.
//
// K and V tiles of BK keys keep their global row layout ([key][D], D*2-byte
// rows, no padding); a row's 16-byte chunks are stored at permuted slots,
// slot = chunk ^ f(row), so that the LDS reads below hit distinct banks.
// The tiles are filled by buffer loads that write LDS directly (each wave
// instruction writes 64 lanes x 16 bytes = RPI whole rows, lane l taking
// slot l % CPR of its row and fetching the chunk that belongs there), so no
// registers stage the tile and no instruction re-packs it.  V is consumed
// through LDS transpose reads (ds_read_b64_tr_b16), which hand each lane
// four consecutive keys of one dimension -- the reduction run an MFMA
// operand needs -- from the natural layout.
// ---------------------------------------------------------------------------
template <int D>
struct Swz {
  static constexpr int CPR = D / 8;        // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;     // rows per 64-lane instruction
  static constexpr int RP = 16 / CPR;      // rows per 256 bytes (one pass over the 64 banks)
  // K: the 16 rows one 16-lane read group touches land on distinct slots
  static __device__ __forceinline__ int fk(int r) { return (r / RP) % CPR; }
  // V: the four consecutive rows a transpose-read group touches land on
  // disjoint 4-chunk blocks
  static __device__ __forceinline__ int fv(int r) { return 4 * ((r / RP) % (4 / RP)); }
};

// This lane's byte offsets (row within the tile, swizzled 16-byte chunk) in
// the tile instructions its wave issues, computed once per workgroup: the
// NT threads share the BK / RPI instructions of a tile, wave w taking
// instructions w, w + W, ...; lane l writes slot l % CPR of row
// RPI * inst + l / CPR and fetches the chunk that belongs there.  When a
// wave's instructions are a whole number of swizzle periods (16 rows)
// apart they share the chunk, and one offset serves them all (the
// instruction's first row goes into its buffer resource).
template <int D, int BK, int NT, bool IS_V>
struct DmaLane {
  typedef Swz<D> S;
  static constexpr int NI = BK / S::RPI, W = NT / 64, PER = NI / W;
  static_assert(NI % W == 0, "tile instructions must split evenly over the waves");
  static constexpr bool SHARED = (S::RPI * W) % 16 == 0;
  int off[SHARED ? 1 : PER];  // relative to the instruction's first row
  __device__ __forceinline__ DmaLane(int row_stride, int tid) {
    const int lane = tid & 63, w = tid >> 6;
#pragma unroll
    for (int x = 0; x < (SHARED ? 1 : PER); ++x) {
      const int r = S::RPI * (w + W * x) + lane / S::CPR;
      const int chunk = (lane % S::CPR) ^ (IS_V ? S::fv(r) : S::fk(r));
      off[x] = (lane / S::CPR) * row_stride * 2 + 16 * chunk;
    }
  }
  __device__ __forceinline__ int get(int x) const { return off[SHARED ? 0 : x]; }
};

// min(max(x, 0), HI) of a uniform x on the scalar unit.  (Written out: the
// compiler otherwise fuses the pair into a vector median instruction and
// then has to move the result back to a scalar register.)
template <int HI>
__device__ __forceinline__ int sclamp_rows(int x) {
  int r;
  __asm__("s_max_i32 %0, %1, 0\n\ts_min_i32 %0, %0, %2" : "=&s"(r) : "s"(x), "n"(HI));
  return r;
}

// Where a request's K or V rows live: base address, bytes per row, row
// count -- uniform values, held in scalar registers.
struct DmaSrc {
  uint32_t lo, hi;
  int row_bytes, n_keys;
};

__device__ __forceinline__ DmaSrc dma_src(const uint16_t* base, int row_stride, int n_keys) {
  const uint64_t a = uint64_t(size_t(base));
  return {uint32_t(__builtin_amdgcn_readfirstlane(int(uint32_t(a)))),
          uint32_t(__builtin_amdgcn_readfirstlane(int(uint32_t(a >> 32)))),
          __builtin_amdgcn_readfirstlane(row_stride * 2), __builtin_amdgcn_readfirstlane(n_keys)};
}

// One BK-key tile (K if IS_V is false, else V), rows key0 .. key0+BK-1 of
// the request at src, into the LDS stage at dst; rows past the request end
// arrive as zeros.  A tile inside the request takes one raw buffer resource
// (gfx9 layout: 48-bit base, stride 0, byte count, 32-bit data format) at
// the wave's first row and a scalar offset per instruction: a handful of
// scalar instructions per tile.  The request's last tile gives each
// instruction a resource of its own over just its rows, cut short at the
// request end, since only the vector offset is range-checked.
// Completion is tracked by vmcnt: the caller waits for it before the
// barrier that publishes the stage.
template <int D, int BK, int NT, bool IS_V>
__device__ __forceinline__ void dma_tile(uint16_t* dst, const DmaSrc& src, int key0,
                                         const DmaLane<D, BK, NT, IS_V>& dl, int tid) {
  typedef DmaLane<D, BK, NT, IS_V> DL;
  typedef Swz<D> S;
  typedef int i32x4 __attribute__((ext_vector_type(4)));
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t lds0 = uint32_t(size_t((__attribute__((address_space(3))) uint16_t*)dst)) + w * 1024;
  const uint64_t base = (uint64_t(src.hi) << 32) | src.lo;
  const int row0 = key0 + S::RPI * w;  // the wave's first row
  // Written as assembly so that the compiler, which cannot tell which LDS
  // bytes a direct-to-LDS load writes, does not make every later LDS read
  // wait for it: the tile goes to a stage no read of the same step
  // touches, and the caller waits (vmcnt) before publishing it.
  if (key0 + BK <= src.n_keys) {
    const uint64_t addr = base + uint64_t(uint32_t(row0)) * uint32_t(src.row_bytes);
    // (readfirstlane: the operands must sit in scalar registers; free when
    // the compiler already keeps them there)
    const i32x4 rsv = {__builtin_amdgcn_readfirstlane(int(uint32_t(addr))),
                       __builtin_amdgcn_readfirstlane(int(uint32_t(addr >> 32) & 0xffffu)),
                       0x7fffffff, 0x00020000};
#pragma unroll
    for (int x = 0; x < DL::PER; ++x) {
      const int soff = __builtin_amdgcn_readfirstlane(S::RPI * DL::W * x * src.row_bytes);
      __asm__ volatile(
          "s_mov_b32 m0, %0\n\t"
          "buffer_load_dwordx4 %1, %2, %3 offen lds"
          :
          : "s"(lds0 + x * DL::W * 1024), "v"(dl.get(x)), "s"(rsv), "s"(soff)
          : "memory", "m0");
    }
  } else {
#pragma unroll
    for (int x = 0; x < DL::PER; ++x) {
      const int rowx = row0 + S::RPI * DL::W * x;  // the instruction's first row
      const uint64_t addr = base + uint64_t(uint32_t(rowx)) * uint32_t(src.row_bytes);
      const i32x4 rsv = {__builtin_amdgcn_readfirstlane(int(uint32_t(addr))),
                         __builtin_amdgcn_readfirstlane(int(uint32_t(addr >> 32) & 0xffffu)),
                         __builtin_amdgcn_readfirstlane(
                             sclamp_rows<S::RPI>(__builtin_amdgcn_readfirstlane(src.n_keys - rowx)) *
                             src.row_bytes),
                         0x00020000};
      __asm__ volatile(
          "s_mov_b32 m0, %0\n\t"
          "buffer_load_dwordx4 %1, %2, 0 offen lds"
          :
          : "s"(lds0 + x * DL::W * 1024), "v"(dl.get(x)), "s"(rsv)
          : "memory", "m0");
    }
  }
}

// One 32-key block of S^T over a swizzled K tile (as qk_block).
template <class T, int D>
__device__ __forceinline__ void qk_block_sw(f32x16& s, const uint16_t* klds, int kb,
                                            const u32x4 (&qb)[D / 16], int lane) {
  typedef typename T::vec8 vec8;
  typedef Swz<D> S;
  const int r = 32 * kb + (lane & 31), h = lane >> 5;
  const uint16_t* row = klds + r * D;
  const int f = S::fk(r);
  f32x16 acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
  for (int u = 0; u < D / 16; ++u) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(row + 8 * ((2 * u + h) ^ f));
    acc = T::mfma32(as<vec8>(a), as<vec8>(qb[u]), acc);
  }
  s = acc;
}

template <class T, int D, int BK, int RB>
__device__ __forceinline__ void qk_tile_sw(f32x16 (&s)[RB][BK / 32], const uint16_t* klds,
                                           const u32x4 (&qb)[RB][D / 16], int lane) {
  typedef typename T::vec8 vec8;
  typedef Swz<D> S;
  const int h = lane >> 5;
#pragma unroll
  for (int kb = 0; kb < BK / 32; ++kb) {
    const int r = 32 * kb + (lane & 31);
    const uint16_t* row = klds + r * D;
    const int f = S::fk(r);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[rb][kb][i] = 0.f;
#pragma unroll
    for (int u = 0; u < D / 16; ++u) {
      const u32x4 a = *reinterpret_cast<const u32x4*>(row + 8 * ((2 * u + h) ^ f));
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        s[rb][kb] = T::mfma32(as<vec8>(a), as<vec8>(qb[rb][u]), s[rb][kb]);
    }
  }
}

// Transposing reads of a swizzled V tile.  Lane q + 4e of each 16-lane group
// supplies the address of row k0 + e, dims dbase + 4q .. +4, and receives
// the four consecutive keys k0 .. k0+3 of dimension dbase + (lane % 16).
// The swizzle of a row repeats every four rows, and every k0 a lane uses is
// 4h plus a multiple of 8, so the address is a per-lane base for each
// 32-dimension block plus a constant: the reads of a tile take D / 32
// address registers and immediate offsets.
template <int D>
__device__ __forceinline__ int vtr_base(int db, int lane) {
  typedef Swz<D> S;
  static_assert(S::RP * (4 / S::RP) == 4, "the V swizzle must repeat every four rows");
  const int i = lane & 15, q = i & 3, e = i >> 2, h = lane >> 5, g2 = (lane >> 4) & 1;
  const int r = 4 * h + e, dim = 32 * db + 16 * g2 + 4 * q;
  return 2 * (r * D + 8 * ((dim >> 3) ^ S::fv(r)) + (dim & 7));
}

__device__ __forceinline__ u32x2 lds_tr4(const uint16_t* vlds, int byte_off) {
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  const char* p = reinterpret_cast<const char*>(vlds) + byte_off;
  const v4i16 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(p));
  return __builtin_bit_cast(u32x2, x);
}

// O^T += V^T P^T over a swizzled V tile.  For score block kb and half t, the
// P operand of lane l (h = l / 32) holds keys 16t + 4h + {0..3} in k-slots
// 0..3 and 16t + 4h + 8 + {0..3} in k-slots 4..7 (the order the S^T
// accumulator hands them over in); two transpose reads give lane l the V
// values of its dimension for exactly those keys.
template <class T, int D, int BK, int RB>
__device__ __forceinline__ void pv_tile_tr(RowState<D> (&st)[RB],
                                           const typename T::vec8 (&pb)[RB][BK / 32][2],
                                           const uint16_t* vlds, int lane) {
  typedef typename T::vec8 vec8;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    const int base = vtr_base<D>(db, lane);
#pragma unroll
    for (int kb = 0; kb < BK / 32; ++kb)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int k0 = 32 * kb + 16 * t;  // plus 4h, inside base
        const u32x2 lo = lds_tr4(vlds, base + 2 * k0 * D);
        const u32x2 hi = lds_tr4(vlds, base + 2 * (k0 + 8) * D);
        const u32x4 a = {lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          st[rb].o[db] = T::mfma32(as<vec8>(a), pb[rb][kb][t], st[rb].o[db]);
      }
  }
}

// Part-tile bitmaps in LDS, re-laid so that one query row's eight bytes are
// adjacent: byte (ir*8 + r)*8 + ic = row r of inner tile (ir, ic), i.e.
// byte r of bitmap word ir*8 + ic (threads 0..63 store word tid).
__device__ __forceinline__ void bitmap_store(uint64_t word, uint8_t* bm, int tid) {
  if (tid < 64) {
    const int ir = tid >> 3, ic = tid & 7;
#pragma unroll
    for (int r = 0; r < 8; ++r) bm[(ir * 8 + r) * 8 + ic] = uint8_t(word >> (8 * r));
  }
}

// Workgroups are dealt to the eight XCDs round robin by linear index, and
// each XCD has its own L2.  With Hq a multiple of 8 the (query block, head)
// grid of the block-sparse kernels is walked so that XCD x serves heads
// x * Hq / 8 .. (x + 1) * Hq / 8 - 1, every query block of them: the K/V of
// those heads stay in that XCD's L2.
__device__ __forceinline__ void bsr_block_head(int nb, int Hq, int& qblk, int& hq) {
  if (Hq & 7) {
    qblk = blockIdx.x;
    hq = blockIdx.y;
    return;
  }
  const int p = blockIdx.x + nb * blockIdx.y, x = p & 7, s = p >> 3;
  hq = x * (Hq >> 3) + s / nb;
  qblk = s % nb;
}

}  // namespace rattn
