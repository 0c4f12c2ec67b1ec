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

// Global -> registers.  Rows key0 .. key0+BK-1 of the request.  On the last
// tile of a request (key0 + BK - 1 > key_last) every row index is clamped to
// key_last, so every address is in bounds; other tiles take the plain path,
// whose per-thread offsets do not depend on the tile and stay in registers.
template <int D, int BK, int NT>
__device__ __forceinline__ void tile_load(TileRegs<D, BK, NT>& rr, const uint16_t* kbase,
                                          const uint16_t* vbase, int64_t row_stride, int key0,
                                          int key_last, int tid) {
  typedef TileRegs<D, BK, NT> R;
  constexpr int CPR = D / 8, HALF = NT / 2;
  const bool tail = key0 + BK - 1 > key_last;
  if (k_role<NT>(tid)) {
    const int t = tid - HALF;
    const uint16_t* kt = kbase + int64_t(key0) * row_stride;
#pragma unroll
    for (int x = 0; x < R::KPT; ++x) {
      const int e = t + HALF * x;
      if (R::KPT * HALF == R::KCHUNKS || e < R::KCHUNKS) {
        int row = e / CPR;
        if (tail) row = key0 + row < key_last ? row : key_last - key0;
        rr.r[x] = ldg128(kt + int64_t(row) * row_stride + 8 * (e % CPR));
      }
    }
  } else {
    const uint16_t* vt = vbase + int64_t(key0) * row_stride;
#pragma unroll
    for (int x = 0; x < R::VPT; ++x) {
      const int e = tid + HALF * x;
      if (R::VPT * HALF == R::VITEMS || e < R::VITEMS) {
        const int kg = e % (BK / 4), dc = e / (BK / 4);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          int row = 4 * kg + b;
          if (tail) row = key0 + row < key_last ? row : key_last - key0;
          rr.r[4 * x + b] = ldg128(vt + int64_t(row) * row_stride + 8 * dc);
        }
      }
    }
  }
}

// Registers -> LDS stage (K natural, V transposed into slot order).
template <int D, int BK, int NT>
__device__ __forceinline__ void tile_store(const TileRegs<D, BK, NT>& rr, uint16_t* lds, int tid) {
  typedef TileGeom<D, BK> Gm;
  typedef TileRegs<D, BK, NT> R;
  constexpr int CPR = D / 8, HALF = NT / 2;
  if (k_role<NT>(tid)) {
    const int t = tid - HALF;
#pragma unroll
    for (int x = 0; x < R::KPT; ++x) {
      const int e = t + HALF * x;
      if (R::KPT * HALF == R::KCHUNKS || e < R::KCHUNKS)
        *reinterpret_cast<u32x4*>(lds + (e / CPR) * Gm::KLD + 8 * (e % CPR)) = rr.r[x];
    }
  } else {
    uint16_t* lv = lds + Gm::K_ELEMS;
#pragma unroll
    for (int x = 0; x < R::VPT; ++x) {
      const int e = tid + HALF * x;
      if (R::VPT * HALF == R::VITEMS || e < R::VITEMS) {
        const int kg = e % (BK / 4), dc = e / (BK / 4);
        // keys 4*kg .. 4*kg+3: T = kg / 4, a = (kg / 2) % 2, h = kg % 2
        const int pos = 16 * (kg >> 2) + 8 * (kg & 1) + 4 * ((kg >> 1) & 1);
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
          *reinterpret_cast<u32x2*>(lv + (8 * dc + jd) * Gm::VLD + pos) = pk;
        }
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

// S^T for one tile: s[kb][r] = q(lane%32) . k(32*kb + 8*(r/4) + 4*h + r%4)
template <class T, int D, int BK>
__device__ __forceinline__ void qk_tile(f32x16 (&s)[BK / 32], const uint16_t* lds,
                                        const u32x4 (&qb)[D / 16], int lane) {
  typedef typename T::vec8 vec8;
  typedef TileGeom<D, BK> Gm;
  const int row = lane & 31, h = lane >> 5;
#pragma unroll
  for (int kb = 0; kb < Gm::NKB; ++kb) {
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
    const uint16_t* kp = lds + (32 * kb + row) * Gm::KLD + 8 * h;
#pragma unroll
    for (int u = 0; u < D / 16; ++u) {
      const u32x4 a = *reinterpret_cast<const u32x4*>(kp + 16 * u);
      acc = T::mfma32(as<vec8>(a), as<vec8>(qb[u]), acc);
    }
    s[kb] = acc;
  }
}

// The running reference max m of a row is raised only when a tile's max
// exceeds it by more than this many log2 units; until then the tile's
// weights exp2(score - m) may reach 2^kRescaleSlack.  The result is the same
// (every weight and the sum share the same reference), but most tiles skip
// the rescale of the output accumulator.
constexpr float kRescaleSlack = 8.f;

// Online softmax, first half: the tile's row max over raw scores s (masked
// entries -inf; c = scale * log2(e) turns a score into log2 units) raises the
// reference max when needed, rescaling O and l.  Returns the reference the
// tile's weights are taken against.
template <int D, int NKB>
__device__ __forceinline__ float softmax_max(RowState<D>& st, const f32x16 (&s)[NKB], float c,
                                             int xaddr) {
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; r += 2) mx = max3(mx, s[kb][r], s[kb][r + 1]);
  mx = fmaxf(mx, swap_halves(mx, xaddr));
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
  // st.m = -inf here means no valid key so far: every s is -inf, p = 0
  return st.m == -INFINITY ? 0.f : st.m;
}

// Second half: the tile's weights exp2(s*c - mref), added to l and returned
// as the bf16/f16 operands pb of the value update.
template <class T, int D, int NKB>
__device__ __forceinline__ void softmax_exp(RowState<D>& st, const f32x16 (&s)[NKB], float c,
                                            float mref, typename T::vec8 (&pb)[NKB][2]) {
  float psum = 0.f;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      f32x8 p;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        p[i] = fexp2(__builtin_fmaf(s[kb][8 * t + i], c, -mref));
        psum += p[i];
      }
      pb[kb][t] = T::cvt8(p);
    }
  st.l += psum;
}

// O^T += V^T P^T over the LDS V^T tile.
template <class T, int D, int BK>
__device__ __forceinline__ void pv_tile(RowState<D>& st, const typename T::vec8 (&pb)[BK / 32][2],
                                        const uint16_t* lds, int lane) {
  typedef typename T::vec8 vec8;
  typedef TileGeom<D, BK> Gm;
  const uint16_t* vp = lds + Gm::K_ELEMS + (lane & 31) * Gm::VLD + 8 * (lane >> 5);
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

template <class T, int D, int BK>
__device__ __forceinline__ void softmax_pv(RowState<D>& st, const f32x16 (&s)[BK / 32], float c,
                                           const uint16_t* lds, int lane) {
  typename T::vec8 pb[BK / 32][2];
  const float mref = softmax_max<D, BK / 32>(st, s, c, (lane ^ 32) << 2);
  softmax_exp<T, D, BK / 32>(st, s, c, mref, pb);
  pv_tile<T, D, BK>(st, pb, lds, lane);
}

// Final normalisation and store of the wave's rows.  orow points at dim 0 of
// this lane's query row (nullptr if the row does not exist); lse_out at its
// LSE slot or nullptr.
template <class T, int D>
__device__ __forceinline__ void row_store(const RowState<D>& st, uint16_t* orow, float* lse_out,
                                          int lane) {
  float l = st.l + swap_halves(st.l, (lane ^ 32) << 2);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const int h = lane >> 5;
  if (orow) {
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
        const typename T::vec8 yb = T::cvt8(y);
        const u32x4 bits = __builtin_bit_cast(u32x4, yb);
        u32x2 out;
        out[0] = bits[0];
        out[1] = bits[1];
        *reinterpret_cast<u32x2*>(orow + 32 * db + 8 * g4 + 4 * h) = out;
      }
  }
  if (lse_out && h == 0) *lse_out = l > 0.f ? (st.m + flog2(l)) * kLn2 : -INFINITY;
}

}  // namespace rattn
