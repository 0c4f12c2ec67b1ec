// decode.hip -- split-KV grouped-query decode on gfx950.
//
// The key dimension of each request is cut by the Split operator into
// chunks of c keys (Cleave article on tip.co.jp, "Split演算子によるSplit-Kの
// 対応"; Cleave arXiv abstract).  One workgroup reduces one
// (chunk, KV head, request) and emits, for each of the G query heads that
// share the KV head, a normalised partial output with its running max and
// sum (m, l).  Inside a chunk the key dimension is tiled (32 keys per wave
// step) and the max and sum reductions run in the same loop over the same
// score tile -- the online softmax that the article's iterative tiling and
// horizontal fusion describe ("複数リダクションのスケジューリング").  A
// second kernel merges the partials with log-sum-exp weights.
//
// Memory: each K/V byte of the request is read exactly once, by the one
// workgroup whose chunk holds it, for all G query heads at once; every
// read is a 16-byte vector load, 16 lanes covering a 256-byte row.
#include "device.hpp"
#include "launch.hpp"


namespace rattn {

// Key range [lo, hi) (offsets inside request b) of split i with chunk c.
// An unused split gets lo >= hi.  Shared by the partial kernels and the
// split-range export so that the export shows what the kernels do.
struct SplitRange {
  int64_t base;  // kv_indptr[b]
  int lo, hi;
};

__device__ __forceinline__ SplitRange split_range(const int32_t* kv_indptr, int b, int i, int c) {
  SplitRange r;
  const int64_t b0 = kv_indptr[b], b1 = kv_indptr[b + 1];
  const int n = int(b1 - b0);
  r.base = b0;
  const int64_t lo = int64_t(i) * c;
  r.lo = lo < n ? int(lo) : n;
  r.hi = lo + c < n ? int(lo + c) : n;
  return r;
}

// -------------------------------------------------------------------------
// MFMA partial kernel (16-bit K/V/Q, fp32 accumulation).
//
// Per wave step the scores of 32 keys against the (up to 16, zero padded)
// query heads are S^T = K Q^T: two 16x16x32 MFMA tiles of 16 keys, the
// head-dimension contraction split into D/32 slabs.  Lane l = (c16, h4)
// (c16 = l % 16, h4 = l / 16) feeds slab u with dims 32u + 8*h4 .. +8 of K
// row (key 16a + c16), so the four lanes of a row read 64 contiguous bytes
// per load instruction.  The accumulator gives lane l head c16 and keys
// 16a + 4*h4 + r.
// The value update is O^T += V^T P^T with 16x16x32 MFMAs: the reduction
// slots of lane (c16, h4) are the keys it already holds scores for,
// kappa(h4, i) = 16*(i/4) + 4*h4 + i%4, so P^T needs no lane exchange;
// MFMA j covers head-dim rows d = (D/16)*rho + j, rho = 0..15, so each
// lane loads D/16 contiguous elements of the rows of its 8 keys (16 lanes
// per 256-byte row) and re-packs them with byte permutes.  Lane (c16, h4)
// ends with head c16, dims (D/4)*h4 .. +D/4 of the output.
// -------------------------------------------------------------------------
template <class T, int D>
struct DecodeTile {
  static constexpr int NU = D / 32;   // QK slabs of 32 dims
  static constexpr int NJ = D / 16;   // PV MFMAs (one per d residue)
  static constexpr int VR = D / 32;   // 32-bit registers per V row piece
  u32x4 k[2][NU];                     // K rows of the two 16-key tiles
  uint32_t v[8][VR];                  // V row pieces of the lane's 8 keys
};

template <class T, int D>
__device__ __forceinline__ void decode_load(DecodeTile<T, D>& t, const uint16_t* kbase,
                                            const uint16_t* vbase, int64_t row_stride,
                                            int key0, int hi, int c16, int h4) {
  constexpr int NU = D / 32;
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    int key = key0 + 16 * a + c16;
    key = key < hi ? key : hi - 1;
    const uint16_t* p = kbase + int64_t(key) * row_stride + 8 * h4;
#pragma unroll
    for (int u = 0; u < NU; ++u) t.k[a][u] = ldg128_nt(p + 32 * u);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    int key = key0 + 16 * (i / 4) + 4 * h4 + (i % 4);
    key = key < hi ? key : hi - 1;
    const uint16_t* p = vbase + int64_t(key) * row_stride + (D / 16) * c16;
    if constexpr (D == 128) {
      u32x4 x = ldg128_nt(p);
      t.v[i][0] = x[0]; t.v[i][1] = x[1]; t.v[i][2] = x[2]; t.v[i][3] = x[3];
    } else {
      u32x2 x = ldg64_nt(p);
      t.v[i][0] = x[0]; t.v[i][1] = x[1];
    }
  }
}

template <class T, int D>
struct DecodeState {
  f32x4 o[D / 16];   // O^T accumulators: o[j][r] is dim (D/4)*h4 + (D/16)*r + j
  float m;           // running max of head c16 (log2 units), same in all 4 h4 lanes
  float l;           // this lane's share of the running sum
};

template <class T, int D>
__device__ __forceinline__ void decode_step(DecodeState<T, D>& st, const DecodeTile<T, D>& t,
                                            const u32x4 (&qb)[D / 32], int key0, int hi,
                                            float sl2, int h4) {
  typedef typename T::vec8 vec8;
  constexpr int NU = D / 32, NJ = D / 16;
  // scores: S^T tiles of 16 keys x 16 heads
  f32x4 s[2];
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    s[a] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < NU; ++u) s[a] = T::mfma16(as<vec8>(t.k[a][u]), as<vec8>(qb[u]), s[a]);
  }
  float x[8];
  const bool tail = key0 + 32 > hi;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float y = s[a][r] * sl2;
      if (tail && key0 + 16 * a + 4 * h4 + r >= hi) y = -INFINITY;
      x[4 * a + r] = y;
    }
  float mx = max3(x[0], x[1], max3(x[2], x[3], max3(x[4], x[5], fmaxf(x[6], x[7]))));
  mx = fmaxf(mx, shfl_xor(mx, 16));
  mx = fmaxf(mx, shfl_xor(mx, 32));
  // every step holds at least one valid key, so mx and m_new are finite
  const float m_new = fmaxf(st.m, mx);
  const float alpha = fexp2(st.m - m_new);
  st.m = m_new;
  f32x8 p;
  float psum = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    p[i] = fexp2(x[i] - m_new);
    psum += p[i];
  }
  st.l = st.l * alpha + psum;
  const vec8 pb = T::cvt8(p);
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    u32x4 a;
    const int w = j / 2;
#pragma unroll
    for (int pr = 0; pr < 4; ++pr)
      a[pr] = (j & 1) ? pack_hi(t.v[2 * pr][w], t.v[2 * pr + 1][w])
                      : pack_lo(t.v[2 * pr][w], t.v[2 * pr + 1][w]);
    st.o[j] *= alpha;
    st.o[j] = T::mfma16(as<vec8>(a), pb, st.o[j]);
  }
}

// Q^T operand of the query heads row0 .. row0 + G - 1 sharing one KV head:
// head c16 (zero past G), slab u -> dims 32u + 8*h4 .. +8.
template <int D>
__device__ __forceinline__ void decode_load_q(u32x4 (&qb)[D / 32], const uint16_t* q, int64_t row0,
                                              int G, int c16, int h4) {
  const uint16_t* qp = q + (row0 + (c16 < G ? c16 : 0)) * D + 8 * h4;
#pragma unroll
  for (int u = 0; u < D / 32; ++u) {
    qb[u] = ldg128(qp + 32 * u);
    if (c16 >= G) qb[u] = u32x4{0u, 0u, 0u, 0u};
  }
}

// The online softmax of one wave over keys 0 .. n-1 of a key range (n >= 1)
// starting at kbase / vbase: 32-key steps ks, ks + WPH, ...  Two register
// buffers: the loads of the next step are in flight while the current one
// is computed.  Loads are issued unconditionally (key indices are clamped
// into the range), so every path leaves the same number of loads
// outstanding and the waits stay exact.  A wave with no step leaves
// st.m = -inf, st.l = 0.
template <class T, int D, int WPH>
__device__ __forceinline__ void decode_range(DecodeState<T, D>& st, const uint16_t* kbase,
                                             const uint16_t* vbase, int64_t row_stride, int n,
                                             int ks, const u32x4 (&qb)[D / 32], float sl2,
                                             int c16, int h4) {
#pragma unroll
  for (int j = 0; j < D / 16; ++j) st.o[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.m = -INFINITY;
  st.l = 0.f;
  const int nsteps = (n + 31) / 32;
  DecodeTile<T, D> t0, t1;
  decode_load<T, D>(t0, kbase, vbase, row_stride, 32 * ks, n, c16, h4);
  for (int s0 = ks; s0 < nsteps; s0 += 2 * WPH) {
    decode_load<T, D>(t1, kbase, vbase, row_stride, 32 * (s0 + WPH), n, c16, h4);
    __builtin_amdgcn_sched_barrier(0);
    decode_step<T, D>(st, t0, qb, 32 * s0, n, sl2, h4);
    if (s0 + WPH >= nsteps) break;
    decode_load<T, D>(t0, kbase, vbase, row_stride, 32 * (s0 + 2 * WPH), n, c16, h4);
    __builtin_amdgcn_sched_barrier(0);
    decode_step<T, D>(st, t1, qb, 32 * (s0 + WPH), n, sl2, h4);
  }
}

// Workgroup = HPW x WPH waves: wave w works on KV head blockIdx.x * HPW +
// w % HPW and takes the 32-key steps w / HPW, w / HPW + WPH, ... of the
// chunk.  Grid (ceil(Hkv / HPW), s, B).
//
// Two shapes are used.  HPW = 4, WPH = 1 (equal request lengths): the
// waves side by side stream the four head slices of the same packed K/V
// rows, so a workgroup reads 1 KB row segments rather than 256-byte pieces
// 2 KB apart -- on MI355X that lifts a plain stream of the decode's reads
// from 5.6 to 6.2 TB/s -- and each wave owns its head's whole chunk, so
// its result needs no combining.  HPW = 1, WPH = 4 (ragged lengths): four
// waves share a head's chunk, so that a chunk, and the tail of the launch
// made of the last chunks, finish four times sooner; the waves' results
// are combined through LDS.
template <class T, int D, int HPW, int WPH>
__global__ __launch_bounds__(64 * HPW * WPH) __attribute__((amdgpu_waves_per_eu(2)))
void decode_partial_mfma(DecodeArgs args) {
  const int w = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  const int hs = w % HPW, ks = w / HPW;
  const int g = blockIdx.x * HPW + hs, i = blockIdx.y, b = blockIdx.z;
  const bool head_ok = g < args.Hkv;  // a last workgroup may hold idle head slots
  const int G = args.G, Hq = args.Hq;
  const int lane = threadIdx.x & 63, c16 = lane & 15, h4 = lane >> 4;
  const int64_t rows = int64_t(args.B) * Hq;
  const SplitRange sr = split_range(args.kv_indptr, b, i, args.chunk);
  const int64_t row0 = int64_t(b) * Hq + int64_t(g) * G;
  if (sr.lo >= sr.hi) {  // split unused by this request (uniform over the workgroup)
    if (!head_ok || ks != 0) return;
    if (args.partials_only) {
      if (lane < G) {
        args.m_part[int64_t(i) * rows + row0 + lane] = -INFINITY;
        args.l_part[int64_t(i) * rows + row0 + lane] = 0.f;
      }
    } else if (i == 0) {    // empty request: O = 0, LSE = -inf
      typename T::elem* o = static_cast<typename T::elem*>(args.o);
      for (int e = lane; e < G * D; e += 64) o[row0 * D + e] = typename T::elem(0.f);
      if (args.lse && lane < G) args.lse[row0 + lane] = -INFINITY;
    }
    return;
  }
  if (WPH == 1 && !head_ok) return;  // no barrier in this shape
  const int gg = head_ok ? g : 0;    // idle slots (WPH > 1) read head 0 and store nothing
  const int64_t row_stride = int64_t(args.Hkv) * D;
  const uint16_t* kbase = static_cast<const uint16_t*>(args.k) + (sr.base + sr.lo) * row_stride +
                          int64_t(gg) * D;
  const uint16_t* vbase = static_cast<const uint16_t*>(args.v) + (sr.base + sr.lo) * row_stride +
                          int64_t(gg) * D;
  const int n = sr.hi - sr.lo;

  u32x4 qb[D / 32];
  decode_load_q<D>(qb, static_cast<const uint16_t*>(args.q), int64_t(b) * Hq + int64_t(gg) * G,
                   G, c16, h4);
  DecodeState<T, D> st;
  decode_range<T, D, WPH>(st, kbase, vbase, row_stride, n, ks, qb, args.scale_log2, c16, h4);

  // lane sums -> head sums (the four h4 lanes of head c16)
  float l = st.l;
  l += shfl_xor(l, 16);
  l += shfl_xor(l, 32);

  // This workgroup's result for its heads: O (normalised), M (log2 units),
  // L.  A request held by a single split is final here; otherwise this is
  // partial i, merged by decode_merge_kernel.
  // (a request longer than s chunks, which a consistent indptr rules out,
  // counts as s splits: its keys past s * chunk are not reduced, and no
  // slot beyond the workspace is ever named)
  const int n_b = int(args.kv_indptr[b + 1] - sr.base);
  int splits_b = args.partials_only ? 0 : (n_b + args.chunk - 1) / args.chunk;
  splits_b = splits_b < args.s ? splits_b : args.s;
  auto emit = [&](int64_t row, int d, float O, float M, float L) {
    if (splits_b == 1) {  // the whole request in one split: final output
      static_cast<typename T::elem*>(args.o)[row * D + d] = typename T::elem(O / L);
      if (d == 0 && args.lse) args.lse[row] = (M + flog2(L)) * kLn2;
    } else {
      args.o_part[(int64_t(i) * rows + row) * D + d] = O / L;
      if (d == 0) {
        args.m_part[int64_t(i) * rows + row] = M * kLn2;
        args.l_part[int64_t(i) * rows + row] = L;
      }
    }
  };
  if constexpr (WPH == 1) {
    // lane (c16, h4) holds dims (D/4)*h4 + (D/16)*r + j of head c16 in o[j][r];
    // st.m is finite (the chunk holds a key)
    if (c16 >= G) return;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int j = 0; j < D / 16; ++j) {
        const int d = (D / 4) * h4 + (D / 16) * r + j;
        emit(row0 + c16, d, st.o[j][r], st.m, l);
      }
  } else {
    // combine the WPH waves of each head through LDS
    __shared__ float red_m[WPH][HPW][16];
    __shared__ float red_l[WPH][HPW][16];
    __shared__ float red_o[WPH][HPW][16][D + 4];
    if (c16 < G) {
      if (h4 == 0) {
        red_m[ks][hs][c16] = st.m;  // -inf for a wave that had no step
        red_l[ks][hs][c16] = l;
      }
#pragma unroll
      for (int j = 0; j < D / 16; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) red_o[ks][hs][c16][(D / 4) * h4 + (D / 16) * r + j] = st.o[j][r];
    }
    __syncthreads();
    for (int e = threadIdx.x; e < HPW * G * D; e += 64 * HPW * WPH) {
      const int slot = e / (G * D), h = (e / D) % G, d = e % D;
      if (blockIdx.x * HPW + slot >= args.Hkv) continue;
      float M = red_m[0][slot][h];
#pragma unroll
      for (int k2 = 1; k2 < WPH; ++k2) M = fmaxf(M, red_m[k2][slot][h]);
      float L = 0.f, O = 0.f;
#pragma unroll
      for (int k2 = 0; k2 < WPH; ++k2) {
        const float f = fexp2(red_m[k2][slot][h] - M);
        L += red_l[k2][slot][h] * f;
        O += red_o[k2][slot][h][d] * f;
      }
      emit(int64_t(b) * Hq + int64_t(blockIdx.x * HPW + slot) * G + h, d, O, M, L);
    }
  }
}

// -------------------------------------------------------------------------
// Flat split plan, for ragged batches.  The Split operator cuts the packed
// key array of the whole batch as one reduction dimension: P pieces of
// c = ceil(total_kv / P) rows, so every workgroup streams the same number of
// key rows whatever the length mix (cutting each request into chunks of
// ceil(max_kv_len / s) keys leaves a launch of unequal last chunks).  Split
// i of request b is its intersection with the i-th piece it overlaps.
//
// Workgroup (x, p) = HPW waves on KV heads x*HPW .. x*HPW + HPW - 1 over
// piece p: side by side the waves read HPW contiguous head slices of each
// packed row (HPW = 4: 1 KB of a 2 KB row of K or V).  A wave walks the
// request segments of its
// piece one after the other with the decode step above; a request lying in
// one piece is final here, the others leave partial i for the merge.
// -------------------------------------------------------------------------
struct FlatSeg {
  int64_t lo, hi;  // packed key rows [lo, hi)
};

// Request rows [r0, r1) inside piece p of c rows.
__device__ __forceinline__ FlatSeg flat_segment(int64_t r0, int64_t r1, int64_t p, int64_t c) {
  const int64_t a = p * c, e = a + c;
  return {r0 > a ? r0 : a, r1 < e ? r1 : e};
}

// Pieces a request of rows [r0, r1) overlaps (0 for an empty request); its
// split i lies in piece r0 / c + i.
__device__ __forceinline__ int flat_splits(int64_t r0, int64_t r1, int64_t c) {
  return r1 > r0 ? int((r1 - 1) / c - r0 / c) + 1 : 0;
}

template <class T, int D, int HPW>
__global__ __launch_bounds__(64 * HPW) __attribute__((amdgpu_waves_per_eu(2)))
void decode_flat_kernel(DecodeArgs args) {
  const int w = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  const int g = blockIdx.x * HPW + w;
  if (g >= args.Hkv) return;  // idle head slot (no barriers in this kernel)
  const int lane = threadIdx.x & 63, c16 = lane & 15, h4 = lane >> 4;
  const int G = args.G, Hq = args.Hq, B = args.B;
  const int64_t rows = int64_t(B) * Hq, c = args.chunk, p = blockIdx.y;
  const int64_t pos0 = p * c;
  const int64_t pos1 = pos0 + c < args.total_kv ? pos0 + c : args.total_kv;
  if (pos0 >= pos1) return;
  // first request that may hold row pos0: (indptr entries <= pos0) - 1,
  // counted 64 entries per step across the lanes
  int cnt = 0;
  for (int j0 = 0; j0 <= B; j0 += 64) {
    const int j = j0 + lane;
    cnt += __popcll(__ballot(j <= B && int64_t(args.kv_indptr[j <= B ? j : B]) <= pos0));
  }
  int b = __builtin_amdgcn_readfirstlane(cnt > 0 ? cnt - 1 : 0);
  const int64_t row_stride = int64_t(args.Hkv) * D;
  for (; b < B; ++b) {
    const int64_t r0 = args.kv_indptr[b], r1 = args.kv_indptr[b + 1];
    if (r0 >= pos1) break;
    const FlatSeg sg = flat_segment(r0, r1, p, c);
    if (sg.lo >= sg.hi) continue;  // empty request, or one that ends before pos0
    const int splits_b = flat_splits(r0, r1, c);
    const int i = int(p - r0 / c);
    // (with a consistent indptr 0 <= i < s always holds; otherwise nothing
    // is written outside the workspace)
    if (splits_b > 1 && (i < 0 || i >= args.s)) continue;
    const int64_t row0 = int64_t(b) * Hq + int64_t(g) * G;
    u32x4 qb[D / 32];
    decode_load_q<D>(qb, static_cast<const uint16_t*>(args.q), row0, G, c16, h4);
    const int64_t off = sg.lo * row_stride + int64_t(g) * D;
    DecodeState<T, D> st;
    decode_range<T, D, 1>(st, static_cast<const uint16_t*>(args.k) + off,
                          static_cast<const uint16_t*>(args.v) + off, row_stride,
                          int(sg.hi - sg.lo), 0, qb, args.scale_log2, c16, h4);
    float l = st.l;
    l += shfl_xor(l, 16);
    l += shfl_xor(l, 32);
    // lane (c16, h4) holds dims (D/4)*h4 + (D/16)*r + j of head c16 in
    // o[j][r]; st.m is finite (the segment holds a key)
    if (c16 < G) {
      const int64_t row = row0 + c16;
      const float inv = 1.f / l;
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int j = 0; j < D / 16; ++j) {
          const int d = (D / 4) * h4 + (D / 16) * r + j;
          if (splits_b == 1)
            static_cast<typename T::elem*>(args.o)[row * D + d] = typename T::elem(st.o[j][r] * inv);
          else
            args.o_part[(int64_t(i) * rows + row) * D + d] = st.o[j][r] * inv;
        }
      if (h4 == 0) {
        if (splits_b == 1) {
          if (args.lse) args.lse[row] = (st.m + flog2(l)) * kLn2;
        } else {
          args.m_part[int64_t(i) * rows + row] = st.m * kLn2;
          args.l_part[int64_t(i) * rows + row] = l;
        }
      }
    }
  }
}

// The flat plan's split ranges, [B, s, 2] key offsets within each request
// (-1 for slots a request does not use), from the same segment arithmetic
// as decode_flat_kernel.
__global__ void flat_ranges_kernel(DecodeArgs a, int32_t* ranges) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= a.B * a.s) return;
  const int b = e / a.s, i = e % a.s;
  const int64_t r0 = a.kv_indptr[b], r1 = a.kv_indptr[b + 1];
  const int64_t c = a.chunk;
  int32_t lo = -1, hi = -1;
  if (c > 0 && i < flat_splits(r0, r1, c)) {
    const FlatSeg sg = flat_segment(r0, r1, r0 / c + i, c);
    lo = int32_t(sg.lo - r0);
    hi = int32_t(sg.hi - r0);
  }
  ranges[2 * e] = lo;
  ranges[2 * e + 1] = hi;
}

// -------------------------------------------------------------------------
// fp32 partial kernel at D = 64 (VALU), for fp32 inputs (small sizes here:
// launch and latency bound).  Workgroup = four waves per (split, KV head, request);
// wave w reduces the key tiles w, w + 4, ... of the split with its own
// online softmax, so that the tiles of a short split run side by side
// rather than one after another.  In a tile of KT keys lane j scores key j
// against the G query heads (the queries staged in LDS), the wave keeps
// per-head running max and sum, and accumulates the value update from the
// tile's V rows, which are loaded (coalesced, 16 bytes per
// lane) at the start of the tile into the wave's own LDS slot, so their
// latency overlaps the key loads and the scores (lane d accumulates output
// dim d).  The four waves' (O, m, l)
// are combined through LDS with log-sum-exp weights.  With one split and
// no partials requested the result is final (O / l and the LSE);
// otherwise it is split i's partial.  GP is G rounded up to a power of two
// (at most 16): the query rows past G are zeros in LDS and every per-head
// loop runs to GP without a branch; only the first G heads are written.
// -------------------------------------------------------------------------
template <int D, int GP>
__global__ __launch_bounds__(256) void decode_partial_f32(DecodeArgs args) {
  constexpr int W = 4;                 // waves per workgroup
  static_assert(D == 64, "D = 128 takes decode_partial_f32_wave");
  constexpr int KT = 64;               // keys per tile (LDS slot of 17 KB per wave)
  constexpr int DL = (D + 63) / 64;    // output dims per lane
  const int i = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int G = args.G, Hq = args.Hq;
  const int64_t rows = int64_t(args.B) * Hq;
  const SplitRange sr = split_range(args.kv_indptr, b, i, args.chunk);
  const int64_t row0 = int64_t(b) * Hq + int64_t(g) * G;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool final_out = args.s == 1 && !args.partials_only;
  if (sr.lo >= sr.hi) {  // unused split, or an empty request (uniform over the workgroup)
    if (tid < G) {
      if (final_out) {  // empty request: O = 0, LSE = -inf
        float* o = static_cast<float*>(args.o) + (row0 + tid) * D;
        for (int d = 0; d < D; ++d) o[d] = 0.f;
        if (args.lse) args.lse[row0 + tid] = -INFINITY;
      } else {
        args.m_part[int64_t(i) * rows + row0 + tid] = -INFINITY;
        args.l_part[int64_t(i) * rows + row0 + tid] = 0.f;
      }
    }
    return;
  }
  __shared__ float qs[GP][D];
  __shared__ float ps[W][KT][GP + 1];
  __shared__ float vs[W][KT][D + 4];  // each wave's tile of V rows
  __shared__ float red_m[W][GP], red_l[W][GP];
  const float* q = static_cast<const float*>(args.q);
  for (int e = tid; e < GP * D; e += 64 * W)
    qs[e / D][e % D] = e < G * D ? q[(row0 + e / D) * D + e % D] : 0.f;
  __syncthreads();
  const int64_t row_stride = int64_t(args.Hkv) * D;
  const float* kb = static_cast<const float*>(args.k) + (sr.base + sr.lo) * row_stride + int64_t(g) * D;
  const float* vb = static_cast<const float*>(args.v) + (sr.base + sr.lo) * row_stride + int64_t(g) * D;
  const int n = sr.hi - sr.lo;
  float m[GP], l[GP], acc[GP][DL];
#pragma unroll
  for (int h = 0; h < GP; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int x = 0; x < DL; ++x) acc[h][x] = 0.f;
  }
  auto wave_sync = [] {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  constexpr int VPL = KT * D / 4 / 64;  // float4 of the V tile per lane
#pragma nounroll
  for (int t0 = KT * w; t0 < n; t0 += KT * W) {
    const int kmax = n - t0 < KT ? n - t0 : KT;
    float4 vreg[VPL];
#pragma unroll
    for (int x = 0; x < VPL; ++x) {
      const int e = x * 64 + lane, r = e / (D / 4), c = e % (D / 4);
      const int rr = r < kmax ? r : kmax - 1;  // rows past the range repeat the last one
      vreg[x] = *reinterpret_cast<const float4*>(vb + int64_t(t0 + rr) * row_stride + 4 * c);
    }
    const bool valid = lane < kmax;
    const float* kr = kb + int64_t(t0 + (valid ? lane : kmax - 1)) * row_stride;
    // The query rows are read from LDS afresh in every tile (their LDS
    // address passes through an empty asm): loop-invariant, they would
    // otherwise be hoisted out of the tile loop into GP * D registers.
    uint32_t qaddr = uint32_t(size_t((__attribute__((address_space(3))) float*)&qs[0][0]));
    __asm__ volatile("" : "+v"(qaddr));
    const __attribute__((address_space(3))) float* qp =
        (const __attribute__((address_space(3))) float*)(size_t)qaddr;
    float sc[GP];
#pragma unroll
    for (int h = 0; h < GP; ++h) sc[h] = 0.f;
#pragma unroll
    for (int d = 0; d < D; d += 4) {
      const float4 kv = *reinterpret_cast<const float4*>(kr + d);
#pragma unroll
      for (int h = 0; h < GP; ++h)
        sc[h] += qp[h * D + d] * kv.x + qp[h * D + d + 1] * kv.y + qp[h * D + d + 2] * kv.z +
                 qp[h * D + d + 3] * kv.w;
    }
#pragma unroll
    for (int h = 0; h < GP; ++h) {
      const float x = valid ? sc[h] * args.scale_log2 : -INFINITY;
      float mx = x;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, shfl_xor(mx, off));
      const float m_new = fmaxf(m[h], mx);  // finite: key t0 is valid
      const float alpha = fexp2(m[h] - m_new);
      const float p = fexp2(x - m_new);
      m[h] = m_new;
      l[h] = l[h] * alpha + p;
#pragma unroll
      for (int xx = 0; xx < DL; ++xx) acc[h][xx] *= alpha;
      if (lane < KT) ps[w][lane][h] = p;
    }
#pragma unroll
    for (int x = 0; x < VPL; ++x) {
      const int e = x * 64 + lane, r = e / (D / 4), c = e % (D / 4);
      *reinterpret_cast<float4*>(&vs[w][r][4 * c]) = vreg[x];
    }
    wave_sync();  // this wave's weights and V rows are in its LDS slot
#pragma unroll 8
    for (int j = 0; j < kmax; ++j) {
#pragma unroll
      for (int xx = 0; xx < DL; ++xx) {
        const float vv = vs[w][j][lane + 64 * xx];
#pragma unroll
        for (int h = 0; h < GP; ++h) acc[h][xx] += ps[w][j][h] * vv;
      }
    }
    wave_sync();  // the slot's reads are done before the next tile's writes
  }
  // combine the waves: m (log2 units, the same in every lane) and the
  // lane-summed l per head, and the unnormalised O rows in the V slots
  // (free once every wave has passed the barrier below)
  __syncthreads();
  float* red_o = &vs[0][0][0];  // [W][GP][D]
  static_assert(W * GP * D <= W * KT * (D + 4), "the waves' rows fit the V slots");
#pragma unroll
  for (int h = 0; h < GP; ++h) {
    float ls = l[h];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ls += shfl_xor(ls, off);
    if (lane == 0) {
      red_m[w][h] = m[h];  // -inf for a wave without a tile
      red_l[w][h] = ls;
    }
#pragma unroll
    for (int xx = 0; xx < DL; ++xx) red_o[(w * GP + h) * D + lane + 64 * xx] = acc[h][xx];
  }
  __syncthreads();
  for (int e = tid; e < G * D; e += 64 * W) {
    const int h = e / D, d = e % D;
    float M = red_m[0][h];
#pragma unroll
    for (int k2 = 1; k2 < W; ++k2) M = fmaxf(M, red_m[k2][h]);  // finite: wave 0 has a tile
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int k2 = 0; k2 < W; ++k2) {
      const float f = fexp2(red_m[k2][h] - M);
      L += red_l[k2][h] * f;
      O += red_o[(k2 * GP + h) * D + d] * f;
    }
    const int64_t row = row0 + h;
    if (final_out) {
      static_cast<float*>(args.o)[row * D + d] = O / L;
      if (d == 0 && args.lse) args.lse[row] = (M + flog2(L)) * kLn2;
    } else {
      args.o_part[(int64_t(i) * rows + row) * D + d] = O / L;
      if (d == 0) {
        args.m_part[int64_t(i) * rows + row] = M * kLn2;
        args.l_part[int64_t(i) * rows + row] = L;
      }
    }
  }
}

// -------------------------------------------------------------------------
// fp32 partial kernel at D = 128 (VALU).  One wave per (split, KV head,
// request), always writing split partials; lane
// j scores key j of each 64-key tile against the G query heads, the wave
// keeps per-head running max and sum, and lane d accumulates output dims d
// and d + 64.  Each tile's V rows are loaded (coalesced, 16 bytes per lane)
// at the start of the tile, so their latency overlaps the key loads and
// the scores, and are read back from LDS by the value update.  Used for
// fp32 inputs, whose sizes here are small (launch and latency bound).
// -------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(64) void decode_partial_f32_wave(DecodeArgs args) {
  constexpr int DL = (D + 63) / 64;  // output dims per lane
  const int i = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int G = args.G, Hq = args.Hq;
  const int64_t rows = int64_t(args.B) * Hq;
  const SplitRange sr = split_range(args.kv_indptr, b, i, args.chunk);
  const int64_t row0 = int64_t(b) * Hq + int64_t(g) * G;
  const int lane = threadIdx.x;
  if (sr.lo >= sr.hi) {
    if (lane < G) {
      args.m_part[int64_t(i) * rows + row0 + lane] = -INFINITY;
      args.l_part[int64_t(i) * rows + row0 + lane] = 0.f;
    }
    return;
  }
  __shared__ float qs[16][D];
  __shared__ float ps[64][17];
  __shared__ float vs[64][D + 4];  // the tile's V rows
  const float* q = static_cast<const float*>(args.q);
  for (int e = lane; e < G * D; e += 64) qs[e / D][e % D] = q[(row0 + e / D) * D + e % D];
  __syncthreads();
  const int64_t row_stride = int64_t(args.Hkv) * D;
  const float* kb = static_cast<const float*>(args.k) + (sr.base + sr.lo) * row_stride + int64_t(g) * D;
  const float* vb = static_cast<const float*>(args.v) + (sr.base + sr.lo) * row_stride + int64_t(g) * D;
  const int n = sr.hi - sr.lo;
  float m[16], l[16], acc[16][DL];
#pragma unroll
  for (int h = 0; h < 16; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int x = 0; x < DL; ++x) acc[h][x] = 0.f;
  }
  constexpr int VPL = D / 4;  // float4 of the V tile per lane
  for (int t0 = 0; t0 < n; t0 += 64) {
    const int kmax = n - t0 < 64 ? n - t0 : 64;
    float4 vreg[VPL];
#pragma unroll
    for (int x = 0; x < VPL; ++x) {
      const int e = x * 64 + lane, r = e / (D / 4), c = e % (D / 4);
      const int rr = r < kmax ? r : kmax - 1;  // rows past the range repeat the last one
      vreg[x] = *reinterpret_cast<const float4*>(vb + int64_t(t0 + rr) * row_stride + 4 * c);
    }
    const int key = t0 + lane;
    const bool valid = key < n;
    const float* kr = kb + int64_t(valid ? key : n - 1) * row_stride;
    float sc[16];
#pragma unroll
    for (int h = 0; h < 16; ++h) sc[h] = 0.f;
#pragma unroll
    for (int d = 0; d < D; d += 4) {
      const float4 kv = *reinterpret_cast<const float4*>(kr + d);
#pragma unroll
      for (int h = 0; h < 16; ++h)
        if (h < G)
          sc[h] += qs[h][d] * kv.x + qs[h][d + 1] * kv.y + qs[h][d + 2] * kv.z + qs[h][d + 3] * kv.w;
    }
#pragma unroll
    for (int h = 0; h < 16; ++h) {
      if (h >= G) break;
      const float x = valid ? sc[h] * args.scale_log2 : -INFINITY;
      float mx = x;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, shfl_xor(mx, off));
      const float m_new = fmaxf(m[h], mx);  // finite: key t0 is valid
      const float alpha = fexp2(m[h] - m_new);
      const float p = fexp2(x - m_new);
      m[h] = m_new;
      l[h] = l[h] * alpha + p;
#pragma unroll
      for (int xx = 0; xx < DL; ++xx) acc[h][xx] *= alpha;
      ps[lane][h] = p;
    }
#pragma unroll
    for (int x = 0; x < VPL; ++x) {
      const int e = x * 64 + lane, r = e / (D / 4), c = e % (D / 4);
      *reinterpret_cast<float4*>(&vs[r][4 * c]) = vreg[x];
    }
    __syncthreads();
    for (int j = 0; j < kmax; ++j) {
#pragma unroll
      for (int xx = 0; xx < DL; ++xx) {
        const int d = lane + 64 * xx;
        if (d < D) {
          const float vv = vs[j][d];
#pragma unroll
          for (int h = 0; h < 16; ++h)
            if (h < G) acc[h][xx] += ps[j][h] * vv;
        }
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int h = 0; h < 16; ++h) {
    if (h >= G) break;
    float ls = l[h];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ls += shfl_xor(ls, off);
    const int64_t row = row0 + h;
#pragma unroll
    for (int xx = 0; xx < DL; ++xx) {
      const int d = lane + 64 * xx;
      if (d < D) args.o_part[(int64_t(i) * rows + row) * D + d] = acc[h][xx] / ls;
    }
    if (lane == 0) {
      args.m_part[int64_t(i) * rows + row] = m[h] * kLn2;
      args.l_part[int64_t(i) * rows + row] = ls;
    }
  }
}

// -------------------------------------------------------------------------
// LSE merge (standalone): one wave per row; lane l holds dims V l .. V l +
// V - 1 (V = D / 64).  The splits' (m, l) -- the first 64 side by side
// across the lanes -- and the partial rows of the first kMergeBatch splits
// are loaded together, then the rest of the partial rows kMergeBatch at a
// time, each batch's loads issued before any is used: one memory round
// trip per batch.  A split with l = 0 (no valid key for the row) has
// weight 0 and its partial row, although loaded, never enters the sum (a
// uniform branch skips it), so whatever an unused slot holds is harmless.
// -------------------------------------------------------------------------
constexpr int kMergeBatch = 8;
template <int D, class OutT, bool H>
__global__ __launch_bounds__(256) void merge_lse_kernel(MergeArgs a) {
  constexpr int V = D / 64;
  const int lane = threadIdx.x & 63;
  // (the wave index read as uniform: the row's indptr entries and split
  // count then live in scalar registers and the loops stay uniform)
  const int64_t row = int64_t(blockIdx.x) * 4 + __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  if (row >= a.rows) return;
  const int64_t rows = a.rows;
  const int s = a.s;
  float x[kMergeBatch][V];
  // partial rows j0 .. j0 + kMergeBatch - 1 of splits [i0, i0 + cnt) (slots
  // past cnt re-read the last one)
  auto load = [&](int i0, int j0, int cnt) {
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) {
      const int jj = j0 + j < cnt ? j0 + j : cnt - 1;
      const int64_t e0 = (int64_t(i0 + jj) * rows + row) * D + V * lane;
      if constexpr (H) {  // fp16 rows; their scale is folded into the weight
        const uint16_t* op = a.o_part16 + e0;
        if constexpr (V == 2) {
          const uint32_t y = *reinterpret_cast<const uint32_t*>(op);
          x[j][0] = F16::to_f32(uint16_t(y));
          x[j][1] = F16::to_f32(uint16_t(y >> 16));
        } else {
          x[j][0] = F16::to_f32(*op);
        }
      } else {
        const float* op = a.o_part + e0;
        if constexpr (V == 2) {
          const float2 y = *reinterpret_cast<const float2*>(op);
          x[j][0] = y.x;
          x[j][1] = y.y;
        } else {
          x[j][0] = *op;
        }
      }
    }
  };
  // the scale of split i's row (lane i of a batch), 1 for fp32 rows
  auto scale_of = [&](int i) { return H ? a.x_part[int64_t(i) * rows + row] : 1.f; };
  float acc[V];
#pragma unroll
  for (int e = 0; e < V; ++e) acc[e] = 0.f;
  auto add = [&](float wi, float xi, int j0, int cnt) {
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) {
      if (j0 + j >= cnt) break;
      const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wi), j0 + j));
      if (wj == 0.f) continue;  // an unused slot: never multiplied
      const float sj = H ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(xi), j0 + j)) : 1.f;
#pragma unroll
      for (int e = 0; e < V; ++e) acc[e] += wj * (H ? x[j][e] * sj : x[j][e]);
    }
  };

  const int cnt0 = s < 64 ? s : 64;
  float mi = -INFINITY, li = 0.f, xi = 1.f;
  if (lane < cnt0) {
    li = a.l_part[int64_t(lane) * rows + row];
    mi = a.m_part[int64_t(lane) * rows + row];
    xi = scale_of(lane);
  }
  if (cnt0 > 0) load(0, 0, cnt0);
  float M = li > 0.f ? mi : -INFINITY;
  for (int i = 64 + lane; i < s; i += 64) {
    const float l2 = a.l_part[int64_t(i) * rows + row];
    if (l2 > 0.f) M = fmaxf(M, a.m_part[int64_t(i) * rows + row]);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, shfl_xor(M, off));
  float wsum = 0.f;
  if (M != -INFINITY) {
    {
      const float wi = li > 0.f ? li * fexp2((mi - M) * kLog2e) : 0.f;
      wsum += wi;
      add(wi, xi, 0, cnt0);
      for (int j0 = kMergeBatch; j0 < cnt0; j0 += kMergeBatch) {
        load(0, j0, cnt0);
        add(wi, xi, j0, cnt0);
      }
    }
    for (int i0 = 64; i0 < s; i0 += 64) {  // more than 64 splits
      const int cnt = s - i0 < 64 ? s - i0 : 64;
      float wi = 0.f, x2 = 1.f;
      if (lane < cnt) {
        const float l2 = a.l_part[int64_t(i0 + lane) * rows + row];
        if (l2 > 0.f) wi = l2 * fexp2((a.m_part[int64_t(i0 + lane) * rows + row] - M) * kLog2e);
        x2 = scale_of(i0 + lane);
      }
      wsum += wi;
      for (int j0 = 0; j0 < cnt; j0 += kMergeBatch) {
        load(i0, j0, cnt);
        add(wi, x2, j0, cnt);
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) wsum += shfl_xor(wsum, off);
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  OutT* o = static_cast<OutT*>(a.o) + row * D + V * lane;
#pragma unroll
  for (int e = 0; e < V; ++e) o[e] = OutT(acc[e] * inv);
  if (a.lse && lane == 0) a.lse[row] = wsum > 0.f ? M + flog2(wsum) * kLn2 : -INFINITY;
}

// -------------------------------------------------------------------------
// Merge inside attn_decode_splitkv: one wave per (request, query head) row.
// The request's split count comes from kv_indptr and the chunk length, so
// rows of requests held by one split (already final) and unused splits are
// never touched; (m, l) of the splits are loaded side by side across lanes.
// -------------------------------------------------------------------------
// D: row width; a wave merges DW = min(D, 128) dims of a row (wider rows,
// such as MLA's 512 latent dims, take D / DW waves).
template <int D, class OutT, int SB>  // SB: splits whose loads are issued together
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeArgs a) {
  constexpr int DW = D < 128 ? D : 128, NSL = D / DW;
  constexpr int DL = (DW + 63) / 64;
  const int lane = threadIdx.x & 63;
  const int64_t rows = int64_t(a.B) * a.Hq;
  // (the wave index read as uniform: the row's indptr entries and split
  // count then live in scalar registers and the loops stay uniform)
  const int64_t gw =
      int64_t(blockIdx.x) * (blockDim.x >> 6) + __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  const int64_t row = gw / NSL;
  const int d0 = int(gw % NSL) * DW;  // this wave's first dim
  if (row >= rows) return;
  const int b = int(row / a.Hq);
  // The request's split count from kv_indptr and the chunk or piece
  // length, capped at the slot count s in both plans, so that no read
  // leaves the workspace even for an indptr inconsistent with max_kv_len;
  // an empty request of the flat plan is written here (O = 0, LSE = -inf)
  // and yields 0.
  const int64_t kb0 = a.kv_indptr[b], kb1 = a.kv_indptr[b + 1];
  auto split_count = [&]() -> int {
    int n;
    if (a.flat) {
      n = a.chunk > 0 ? flat_splits(kb0, kb1, a.chunk) : 0;
      n = n < a.s ? n : a.s;
      if (n == 0) {
        OutT* o = static_cast<OutT*>(a.o) + row * D + d0;
#pragma unroll
        for (int x = 0; x < DL; ++x)
          if (lane + 64 * x < DW) o[lane + 64 * x] = OutT(0.f);
        if (a.lse && lane == 0 && d0 == 0) a.lse[row] = -INFINITY;
      }
    } else {
      n = a.chunk > 0 ? int((kb1 - kb0 + a.chunk - 1) / a.chunk) : 0;
      n = n < a.s ? n : a.s;
    }
    return n;
  };
  // The first n splits' (m, l) and partial outputs, loaded at once.
  float mi = -INFINITY, li = 0.f;
  float ov[SB][DL];
  auto load_batch = [&](int n) {
    if (lane < n) {
      mi = a.m_part[int64_t(lane) * rows + row];
      li = a.l_part[int64_t(lane) * rows + row];
    }
#pragma unroll
    for (int j = 0; j < SB; ++j)
#pragma unroll
      for (int x = 0; x < DL; ++x)
        ov[j][x] = (j < n && lane + 64 * x < DW) ? a.o_part[(int64_t(j) * rows + row) * D + d0 + lane + 64 * x] : 0.f;
  };
  int splits_b;
  if (a.uniform) {
    // equal lengths: every request uses min(s, SB) of the first slots, so
    // the loads go out together with the indptr reads (one round trip)
    load_batch(a.s < SB ? a.s : SB);
    splits_b = split_count();
  } else {
    // ragged: only the request's own splits are loaded
    splits_b = split_count();
    if (splits_b > 1) load_batch(splits_b < SB ? splits_b : SB);
  }
  if (splits_b <= 1) return;
  if (lane >= splits_b) { mi = -INFINITY; li = 0.f; }
  float M = mi;
  for (int i = SB + lane; i < splits_b; i += 64) M = fmaxf(M, a.m_part[int64_t(i) * rows + row]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, shfl_xor(M, off));
  float acc[DL];
#pragma unroll
  for (int x = 0; x < DL; ++x) acc[x] = 0.f;
  float wsum = 0.f;
  {
    // splits 0 .. SB-1 from the registers loaded above
    const float wi = lane < splits_b ? li * fexp2((mi - M) * kLog2e) : 0.f;
    float ws = wi;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ws += shfl_xor(ws, off);
    wsum += ws;
#pragma unroll
    for (int j = 0; j < SB; ++j) {
      const float wj = __shfl(wi, j, 64);
      if (j < splits_b) {
#pragma unroll
        for (int x = 0; x < DL; ++x) acc[x] += wj * ov[j][x];
      }
    }
  }
  // splits SB .. splits_b-1, if any, in batches of 64
  for (int i0 = SB; i0 < splits_b; i0 += 64) {
    float wi = 0.f;
    if (i0 + lane < splits_b) {
      const float m2 = a.m_part[int64_t(i0 + lane) * rows + row];
      const float l2 = a.l_part[int64_t(i0 + lane) * rows + row];
      wi = l2 * fexp2((m2 - M) * kLog2e);
    }
    float ws = wi;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ws += shfl_xor(ws, off);
    wsum += ws;
    const int n = splits_b - i0 < 64 ? splits_b - i0 : 64;
    const float* op = a.o_part + (int64_t(i0) * rows + row) * D + d0 + lane;
#pragma unroll 4
    for (int j = 0; j < n; ++j) {
      const float wj = __shfl(wi, j, 64);
#pragma unroll
      for (int x = 0; x < DL; ++x)
        if (lane + 64 * x < DW) acc[x] += wj * op[int64_t(j) * rows * D + 64 * x];
    }
  }
  const float inv = 1.f / wsum;
  OutT* o = static_cast<OutT*>(a.o) + row * D + d0;
#pragma unroll
  for (int x = 0; x < DL; ++x) {
    const int d = lane + 64 * x;
    if (d < DW) o[d] = OutT(acc[x] * inv);
  }
  if (a.lse && lane == 0 && d0 == 0) a.lse[row] = M + flog2(wsum) * kLn2;
}

__global__ void split_ranges_kernel(const int32_t* kv_indptr, int B, int s, int chunk,
                                    int32_t* ranges) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= B * s) return;
  const int b = e / s, i = e % s;
  const SplitRange sr = split_range(kv_indptr, b, i, chunk);
  ranges[2 * e] = sr.lo < sr.hi ? sr.lo : -1;
  ranges[2 * e + 1] = sr.lo < sr.hi ? sr.hi : -1;
}

// ---- launchers -----------------------------------------------------------

// Workgroup shape: four waves side by side on four KV heads when every
// request has the same length (the host passes uniform = 1), one KV head
// with four waves splitting its chunk otherwise.  Heads per workgroup never
// exceed Hkv.
template <class T, int D>
static void launch_partial_mfma_t(const DecodeArgs& a, hipStream_t st) {
  const int hpw = a.uniform ? (a.Hkv >= 4 ? 4 : a.Hkv >= 2 ? 2 : 1) : 1;
  const dim3 grid(unsigned((a.Hkv + hpw - 1) / hpw), unsigned(a.s), unsigned(a.B));
  switch (hpw) {
    case 4: hipLaunchKernelGGL((decode_partial_mfma<T, D, 4, 1>), grid, dim3(256), 0, st, a); break;
    case 2: hipLaunchKernelGGL((decode_partial_mfma<T, D, 2, 1>), grid, dim3(128), 0, st, a); break;
    default:
      if (a.uniform) hipLaunchKernelGGL((decode_partial_mfma<T, D, 1, 1>), grid, dim3(64), 0, st, a);
      else hipLaunchKernelGGL((decode_partial_mfma<T, D, 1, 4>), grid, dim3(256), 0, st, a);
      break;
  }
}

static void launch_partial_mfma(const DecodeArgs& a, hipStream_t st) {
  if (a.dtype == 1) {
    if (a.D == 64) launch_partial_mfma_t<BF16, 64>(a, st); else launch_partial_mfma_t<BF16, 128>(a, st);
  } else {
    if (a.D == 64) launch_partial_mfma_t<F16, 64>(a, st); else launch_partial_mfma_t<F16, 128>(a, st);
  }
}

// fp32 partial kernel at D = 64 at the padded head count of G (1, 2, 4, 8
// or 16)
template <int D>
static void launch_partial_f32_d(const DecodeArgs& a, hipStream_t st) {
  const dim3 grid(a.s, a.Hkv, a.B), block(256);
  if (a.G <= 1) hipLaunchKernelGGL((decode_partial_f32<D, 1>), grid, block, 0, st, a);
  else if (a.G <= 2) hipLaunchKernelGGL((decode_partial_f32<D, 2>), grid, block, 0, st, a);
  else if (a.G <= 4) hipLaunchKernelGGL((decode_partial_f32<D, 4>), grid, block, 0, st, a);
  else if (a.G <= 8) hipLaunchKernelGGL((decode_partial_f32<D, 8>), grid, block, 0, st, a);
  else hipLaunchKernelGGL((decode_partial_f32<D, 16>), grid, block, 0, st, a);
}

// D = 128: the one-wave kernel, which always writes split partials
static void launch_partial_f32(const DecodeArgs& a, hipStream_t st) {
  if (a.D == 64) launch_partial_f32_d<64>(a, st);
  else hipLaunchKernelGGL(decode_partial_f32_wave<128>, dim3(a.s, a.Hkv, a.B), dim3(64), 0, st, a);
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t st) {
  const dim3 grid(a.s, a.Hkv, a.B);
  if (a.dtype == 0) {  // fp32: partial kernel, then (s > 1) the standalone merge
    launch_partial_f32(a, st);
    hipError_t e = hipGetLastError();
    // one split at D = 64: the kernel's result is final
    if (e != hipSuccess || (a.s == 1 && a.D == 64)) return e;
    MergeArgs m{a.o_part, a.m_part, a.l_part, a.s, a.B * a.Hq, a.D, a.o, 0, a.lse};
    return launch_merge(m, st);
  } else {  // 16-bit: MFMA partial kernel, then the merge of multi-split requests
    launch_partial_mfma(a, st);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.s == 1) return e;  // one split: every request is final
    // equal lengths: every request has s splits, loaded in one batch of 8
    // (s <= 8) or 16; ragged: up to 32 of a request's own splits
    // two rows (waves) per workgroup: on MI355X the step ran 0.7-0.9 us
    // shorter than with four
    const dim3 mgrid(unsigned((int64_t(a.B) * a.Hq + 1) / 2));
#define RATTN_MERGE(DD, TT)                                                                  \
  if (a.uniform && a.s <= 8) hipLaunchKernelGGL((decode_merge_kernel<DD, TT, 8>), mgrid, dim3(128), 0, st, a); \
  else if (a.uniform) hipLaunchKernelGGL((decode_merge_kernel<DD, TT, 16>), mgrid, dim3(128), 0, st, a); \
  else hipLaunchKernelGGL((decode_merge_kernel<DD, TT, 32>), mgrid, dim3(128), 0, st, a)
    if (a.dtype == 1) {
      if (a.D == 64) { RATTN_MERGE(64, __bf16); } else { RATTN_MERGE(128, __bf16); }
    } else {
      if (a.D == 64) { RATTN_MERGE(64, _Float16); } else { RATTN_MERGE(128, _Float16); }
    }
#undef RATTN_MERGE
  }
  return hipGetLastError();
}

// Up to four KV heads per workgroup: on MI355X a piece streamed by four
// waves side by side (1 KB of each 2 KB packed row) at one workgroup per
// compute unit sustained more than eight waves on whole rows, or two.
template <class T, int D>
static void launch_flat_t(const DecodeArgs& a, hipStream_t st) {
  const int hpw = a.Hkv >= 4 ? 4 : a.Hkv >= 2 ? 2 : 1;
  const dim3 grid(unsigned((a.Hkv + hpw - 1) / hpw), unsigned(a.pieces));
  if (a.pieces > 0 && a.total_kv > 0) switch (hpw) {
    case 4: hipLaunchKernelGGL((decode_flat_kernel<T, D, 4>), grid, dim3(256), 0, st, a); break;
    case 2: hipLaunchKernelGGL((decode_flat_kernel<T, D, 2>), grid, dim3(128), 0, st, a); break;
    default: hipLaunchKernelGGL((decode_flat_kernel<T, D, 1>), grid, dim3(64), 0, st, a); break;
  }
  const dim3 mgrid(unsigned((int64_t(a.B) * a.Hq + 1) / 2));
  hipLaunchKernelGGL((decode_merge_kernel<D, typename T::elem, 32>), mgrid, dim3(128), 0, st, a);
}

hipError_t launch_decode_flat(const DecodeArgs& a, hipStream_t st) {
  if (a.dtype == 1) {
    if (a.D == 64) launch_flat_t<BF16, 64>(a, st); else launch_flat_t<BF16, 128>(a, st);
  } else {
    if (a.D == 64) launch_flat_t<F16, 64>(a, st); else launch_flat_t<F16, 128>(a, st);
  }
  return hipGetLastError();
}

hipError_t launch_flat_ranges(const DecodeArgs& a, int32_t* ranges, hipStream_t st) {
  const int n = a.B * a.s;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(flat_ranges_kernel, dim3((n + 255) / 256), dim3(256), 0, st, a, ranges);
  return hipGetLastError();
}

hipError_t launch_decode_partials(const DecodeArgs& a, hipStream_t st) {
  const dim3 grid(a.s, a.Hkv, a.B);
  if (a.dtype == 0) {
    launch_partial_f32(a, st);
  } else {
    launch_partial_mfma(a, st);
  }
  return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t st) {
  const dim3 grid((a.rows + 3) / 4);
  if (a.rows == 0) return hipSuccess;
#define RATTN_MERGE(DD, TT)                                                                    \
  do {                                                                                         \
    if (a.o_part16) hipLaunchKernelGGL((merge_lse_kernel<DD, TT, true>), grid, dim3(256), 0, st, a); \
    else hipLaunchKernelGGL((merge_lse_kernel<DD, TT, false>), grid, dim3(256), 0, st, a);     \
  } while (0)
  if (a.D == 64) {
    if (a.o_dtype == 0) RATTN_MERGE(64, float);
    else if (a.o_dtype == 1) RATTN_MERGE(64, __bf16);
    else RATTN_MERGE(64, _Float16);
  } else {
    if (a.o_dtype == 0) RATTN_MERGE(128, float);
    else if (a.o_dtype == 1) RATTN_MERGE(128, __bf16);
    else RATTN_MERGE(128, _Float16);
  }
#undef RATTN_MERGE
  return hipGetLastError();
}

hipError_t launch_split_ranges(const int32_t* kv_indptr, int B, int s, int chunk, int32_t* ranges,
                               hipStream_t st) {
  const int n = B * s;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(split_ranges_kernel, dim3((n + 255) / 256), dim3(256), 0, st, kv_indptr, B, s,
                     chunk, ranges);
  return hipGetLastError();
}

}  // namespace rattn
