// attn_core.hpp -- the fused attention tile step shared by the dense/causal
// prefill kernel and the block-sparse kernel (gfx950, 32x32x16 MFMA).
//
// One wave owns 32 query rows.  Keys arrive in tiles of 64 staged in LDS
// (iterative tiling of the key dimension, Cleave article on tip.co.jp,
// "複数リダクションのスケジューリング"); for each tile the wave computes the
// transposed score block S^T = K Q^T, updates the row max and the row sum of
// exp over that same block in one pass (horizontal fusion), rescales its
// output accumulator and adds V^T P^T.  Working on S^T puts one query per
// lane column, so each row's max and sum are lane-local plus a single
// exchange with the partner lane l ^ 32.
//
// LDS layout per stage:
//   K tile  [64 keys][D + 8] (natural row order; +16 B pad per row spreads
//           the 32 rows one MFMA operand read touches over all banks)
//   V^T tile [D][64 + 8] with keys stored in "slot order":
//           key k = 16*T + 8*a + 4*h + b  ->  position 16*T + 8*h + 4*a + b,
//           so that the eight reduction slots lane half h feeds to one
//           V^T P^T MFMA are 16 contiguous bytes.
#pragma once
#include "device.hpp"

namespace rattn {

template <int D>
struct TileGeom {
  static constexpr int BK = 64;           // keys per tile
  static constexpr int KLD = D + 8;       // K row stride (elements)
  static constexpr int VLD = BK + 8;      // V^T row stride (elements)
  static constexpr int K_ELEMS = BK * KLD;
  static constexpr int V_ELEMS = D * VLD;
  static constexpr int STAGE = K_ELEMS + V_ELEMS;  // 16-bit elements per stage
};

// Registers holding one K/V tile between its global load and its LDS store.
template <int D, int NT>
struct TileRegs {
  static constexpr int KCH = 64 * (D / 8) / NT;               // 16-byte K chunks per thread
  static constexpr int VIT = (16 * (D / 8) + NT - 1) / NT;    // (4 keys x 8 dims) V items per thread
  u32x4 k[KCH];
  u32x4 v[VIT][4];
};

// Global -> registers.  Rows key0 .. key0+63 of the request, each clamped to
// key_last (the last row that exists), so every address is in bounds.
template <int D, int NT>
__device__ __forceinline__ void tile_load(TileRegs<D, NT>& r, const uint16_t* kbase,
                                          const uint16_t* vbase, int64_t row_stride, int key0,
                                          int key_last, int tid) {
  constexpr int CPR = D / 8;  // chunks per row
#pragma unroll
  for (int x = 0; x < TileRegs<D, NT>::KCH; ++x) {
    const int e = tid + NT * x;
    int key = key0 + e / CPR;
    key = key < key_last ? key : key_last;
    r.k[x] = ldg128(kbase + int64_t(key) * row_stride + 8 * (e % CPR));
  }
#pragma unroll
  for (int x = 0; x < TileRegs<D, NT>::VIT; ++x) {
    const int e = tid + NT * x;
    if (e < 16 * CPR) {
      const int kg = e & 15, dc = e >> 4;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        int key = key0 + 4 * kg + b;
        key = key < key_last ? key : key_last;
        r.v[x][b] = ldg128(vbase + int64_t(key) * row_stride + 8 * dc);
      }
    }
  }
}

// Registers -> LDS stage (K natural, V transposed into slot order).
template <int D, int NT>
__device__ __forceinline__ void tile_store(const TileRegs<D, NT>& r, uint16_t* lds, int tid) {
  typedef TileGeom<D> Gm;
  constexpr int CPR = D / 8;
  uint16_t* lk = lds;
  uint16_t* lv = lds + Gm::K_ELEMS;
#pragma unroll
  for (int x = 0; x < TileRegs<D, NT>::KCH; ++x) {
    const int e = tid + NT * x;
    *reinterpret_cast<u32x4*>(lk + (e / CPR) * Gm::KLD + 8 * (e % CPR)) = r.k[x];
  }
#pragma unroll
  for (int x = 0; x < TileRegs<D, NT>::VIT; ++x) {
    const int e = tid + NT * x;
    if (e < 16 * CPR) {
      const int kg = e & 15, dc = e >> 4;
      // keys 4*kg .. 4*kg+3: T = kg / 4, a = (kg / 2) % 2, h = kg % 2
      const int pos = 16 * (kg >> 2) + 8 * (kg & 1) + 4 * ((kg >> 1) & 1);
#pragma unroll
      for (int jd = 0; jd < 8; ++jd) {
        const int w = jd >> 1;
        u32x2 pk;
        if (jd & 1) {
          pk[0] = pack_hi(r.v[x][0][w], r.v[x][1][w]);
          pk[1] = pack_hi(r.v[x][2][w], r.v[x][3][w]);
        } else {
          pk[0] = pack_lo(r.v[x][0][w], r.v[x][1][w]);
          pk[1] = pack_lo(r.v[x][2][w], r.v[x][3][w]);
        }
        *reinterpret_cast<u32x2*>(lv + (8 * dc + jd) * Gm::VLD + pos) = pk;
      }
    }
  }
}

// Per-wave running state of 32 query rows (one per lane column).
template <int D>
struct RowState {
  f32x16 o[D / 32];  // O^T accumulators: o[db][r] is dim 32*db + 8*(r/4) + 4*h + r%4
  float m;           // running max (log2 units), equal in lanes l and l^32
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
template <int D>
__device__ __forceinline__ void load_q(u32x4 (&qb)[D / 16], const uint16_t* qrow, int lane) {
  const int h = lane >> 5;
#pragma unroll
  for (int u = 0; u < D / 16; ++u) qb[u] = ldg128(qrow + 16 * u + 8 * h);
}

// S^T for the 64-key tile: s[kb][r] = q(lane%32) . k(32*kb + 8*(r/4) + 4*h + r%4)
template <class T, int D>
__device__ __forceinline__ void qk_tile(f32x16 (&s)[2], const uint16_t* lds,
                                        const u32x4 (&qb)[D / 16], int lane) {
  typedef typename T::vec8 vec8;
  typedef TileGeom<D> Gm;
  const int row = lane & 31, h = lane >> 5;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
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

// Online softmax update over the scaled, masked scores x (log2 units), then
// O^T += V^T P^T from the LDS V^T tile.
template <class T, int D>
__device__ __forceinline__ void softmax_pv(RowState<D>& st, float (&x)[2][16], const uint16_t* lds,
                                           int lane) {
  typedef typename T::vec8 vec8;
  typedef TileGeom<D> Gm;
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; r += 2) mx = max3(mx, x[kb][r], x[kb][r + 1]);
  mx = fmaxf(mx, shfl_xor(mx, 32));
  const float m_new = fmaxf(st.m, mx);
  const float m_use = m_new == -INFINITY ? 0.f : m_new;  // row fully masked so far
  const float alpha = fexp2(st.m - m_use);
  st.m = m_new;
  float psum = 0.f;
  vec8 pb[2][2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      f32x8 p;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        p[i] = fexp2(x[kb][8 * t + i] - m_use);
        psum += p[i];
      }
      pb[kb][t] = T::cvt8(p);
    }
  st.l = st.l * alpha + psum;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) st.o[db] *= alpha;
  const uint16_t* vp = lds + Gm::K_ELEMS + (lane & 31) * Gm::VLD + 8 * (lane >> 5);
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(vp + 32 * db * Gm::VLD + 32 * kb + 16 * t);
        st.o[db] = T::mfma32(as<vec8>(a), pb[kb][t], st.o[db]);
      }
}

// Final normalisation and store of the wave's rows.  orow points at dim 0 of
// this lane's query row (nullptr if the row does not exist); lse_out at its
// LSE slot or nullptr.
template <class T, int D>
__device__ __forceinline__ void row_store(const RowState<D>& st, uint16_t* orow, float* lse_out,
                                          int lane) {
  float l = st.l + shfl_xor(st.l, 32);
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
