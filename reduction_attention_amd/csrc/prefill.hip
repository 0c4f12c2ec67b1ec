// prefill.hip -- fused prefill attention on gfx950: dense / causal over a
// ragged batch, and block-sparse over STOF's two-level mask.
//
// Both kernels stream key/value tiles of 64 keys through LDS while the query
// tile stays in registers, and fuse QK^T, the row max, the exp-sum and PV
// into one loop (attn_core.hpp).  The dense kernel
// follows the iterative tiling and horizontal fusion of the Cleave article
// (tip.co.jp, "複数リダクションのスケジューリング"), with dynamic batch and
// sequence lengths read from indptr arrays at run time so one compiled
// kernel serves every shape (same section, last paragraph).  The sparse
// kernel is the block-wise kernel of the STOF explainer (gist.science,
// 技術概要, "1. 統合 MHA モジュール", "デュアルカーネル戦略"): it visits only the
// stored outer tiles of its query block row, skips the element test on
// full tiles and applies the 8x8 inner-tile bitmaps on part tiles.
#include "attn_core.hpp"
#include "launch.hpp"

namespace rattn {

// ---------------------------------------------------------------------------
// Dense / causal prefill.  Workgroup = W waves, each owning RB blocks of 32
// query rows of one query head; grid (Hq, B, query tiles), causal tiles
// issued heaviest first, two workgroups per compute unit.
//
// Keys arrive in tiles of BK.  In step j a wave computes the scores of tile
// j + 1 and the value update of tile j (weights from the previous step),
// then the weights of tile j + 1.  K therefore runs one tile ahead of V:
// LDS holds two K stages and two V stages (64 KB at D = 128), and the tiles
// issued at the top of step j (K of tile j + 2, V of tile j + 1) stream
// straight from memory into the stages step j - 1 released while the step
// computes; one wait and one barrier end the step.  Tiles keep their
// natural layout with swizzled 16-byte slots; V is read through transposing
// LDS reads (attn_core.hpp).  Two workgroups share a compute unit, so one's
// start-up (its query rows and first tiles coming in from memory) and
// barriers overlap the other's matrix work.  The shape below (waves per
// workgroup, 32-row blocks per wave, workgroups per compute unit, keys per
// tile) won a sweep on MI355X against 8 waves, two row blocks per wave, one
// workgroup per compute unit and 32- or 128-key tiles.
// ---------------------------------------------------------------------------
constexpr int kPrefillWaves = 4;
constexpr int kPrefillRB = 1;
constexpr int kPrefillOcc = 2;
constexpr int kPrefillBK = 64;
constexpr int kPrefillBQ = 32 * kPrefillRB * kPrefillWaves;  // query rows per workgroup

// Workgroups are dealt to the eight XCDs round robin by linear index, and
// each XCD has its own L2.  With Hq a multiple of 8, grid column x runs head
// (x % 8) * (Hq / 8) + x / 8, so each XCD serves a contiguous range of query
// heads -- whole GQA groups -- and fetches their K/V into its own L2 only.
__device__ __forceinline__ int xcd_head(int x, int hq_count) {
  if (hq_count & 7) return x;
  return (x & 7) * (hq_count >> 3) + (x >> 3);
}

// The value update's schedule: N matrix ops (times RB), each fed by two
// transposing LDS reads, with kPvDepth reads kept in flight ahead of them.
constexpr int kPvDepth = 8;
template <int N, int RB>
__device__ __forceinline__ void lds_pipeline_pv() {
  __builtin_amdgcn_sched_group_barrier(0x100, kPvDepth, 1);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, RB, 1);
    if (i < N - kPvDepth / 2) __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
  }
}

// Schedule of a block of N operand reads from LDS, each feeding RB matrix
// ops: keep kLdsDepth reads in flight ahead of the matrix ops (two, three
// and five measured no better than four).
constexpr int kLdsDepth = 4;
template <int N, int RB>
__device__ __forceinline__ void lds_pipeline() {
  __builtin_amdgcn_sched_group_barrier(0x100, kLdsDepth, 0);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, RB, 0);
    if (i + kLdsDepth < N) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
}

template <class T, int D, bool CAUSAL>
__global__ __launch_bounds__(64 * kPrefillWaves, kPrefillOcc)
void prefill_kernel(PrefillArgs a) {
  constexpr int NT = 64 * kPrefillWaves, RB = kPrefillRB, BQ = kPrefillBQ, BK = kPrefillBK;
  typedef TileGeom<D, BK> Gm;
  typedef typename T::vec8 vec8;
  constexpr int TE = BK * D;  // elements per natural-layout tile
  __shared__ __attribute__((aligned(16))) uint16_t lds_k[2 * TE];
  __shared__ __attribute__((aligned(16))) uint16_t lds_v[2 * TE];
  uint16_t* const lds_k0 = lds_k;
  uint16_t* const lds_k1 = lds_k + TE;
  uint16_t* const lds_v0 = lds_v;
  uint16_t* const lds_v1 = lds_v + TE;

  // grid (Hq, B, query tiles x splits): workgroups are dispatched in linear
  // order, so with the query tile slowest every causal tile of one size
  // goes out before any smaller one (heaviest first) and the short ones
  // fill the tail.  Split si covers keys [si * chunk, (si + 1) * chunk).
  const int hq = xcd_head(blockIdx.x, a.Hq), b = blockIdx.y;
  const int nqt = int(gridDim.z) / a.s;
  const int zq = int(blockIdx.z) / a.s, si = int(blockIdx.z) % a.s;
  const int qt = CAUSAL ? nqt - 1 - zq : zq;
  const int64_t q_begin = a.qo_indptr[b];
  const int n_q = int(a.qo_indptr[b + 1] - q_begin);
  const int64_t k_begin = a.kv_indptr[b];
  const int n_kv = int(a.kv_indptr[b + 1] - k_begin);
  const int q_start = qt * BQ;
  if (q_start >= n_q) return;
  const int k_lo = a.s > 1 ? si * a.chunk : 0;
  const int k_hi = a.s > 1 ? (k_lo + a.chunk < n_kv ? k_lo + a.chunk : n_kv) : n_kv;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
  const int g = hq / a.G;
  const int off = n_kv - n_q;  // causal: key j valid for query i iff j <= i + off
  const int q_last_wg = (q_start + BQ < n_q ? q_start + BQ : n_q) - 1;
  int kv_end = k_hi;
  if (CAUSAL) kv_end = q_last_wg + 1 + off < k_hi ? q_last_wg + 1 + off : k_hi;
  const int ntiles = kv_end > k_lo ? (kv_end - k_lo + BK - 1) / BK : 0;

  // this wave's rows (RB blocks of 32) and the tiles it takes part in
  const int q0w = q_start + 32 * RB * w;
  int wnt = 0;
  if (q0w < n_q) {
    const int wq_last = q0w + 32 * RB - 1 < n_q ? q0w + 32 * RB - 1 : n_q - 1;
    int wkv_end = k_hi;
    if (CAUSAL) wkv_end = wq_last + 1 + off < k_hi ? wq_last + 1 + off : k_hi;
    wnt = wkv_end > k_lo ? (wkv_end - k_lo + BK - 1) / BK : 0;
  }
  wnt = __builtin_amdgcn_readfirstlane(wnt);
  const uint16_t* Q = static_cast<const uint16_t*>(a.q);
  u32x4 qb[RB][D / 16];
  RowState<D> st[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int mq = q0w + 32 * rb + (lane & 31);
    load_q<D>(qb[rb], Q + ((q_begin + (mq < n_q ? mq : n_q - 1)) * a.Hq + hq) * D, lane);
    row_state_init(st[rb]);
  }
  const float c = a.scale_log2;

  const int row_stride = a.Hkv * D;
  const uint16_t* kbase = static_cast<const uint16_t*>(a.k) + k_begin * row_stride + int64_t(g) * D;
  const uint16_t* vbase = static_cast<const uint16_t*>(a.v) + k_begin * row_stride + int64_t(g) * D;
  const DmaSrc ksrc = dma_src(kbase, row_stride, n_kv), vsrc = dma_src(vbase, row_stride, n_kv);

  // prologue: K of tiles 0 and 1, V of tile 0
  const DmaLane<D, BK, NT, false> dk(row_stride, tid);
  const DmaLane<D, BK, NT, true> dv(row_stride, tid);
  if (ntiles > 0) {
    dma_tile<D, BK, NT, false>(lds_k0, ksrc, k_lo, dk, tid);
    dma_tile<D, BK, NT, true>(lds_v0, vsrc, k_lo, dv, tid);
  }
  if (ntiles > 1) dma_tile<D, BK, NT, false>(lds_k1, ksrc, k_lo + BK, dk, tid);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the tiles are in LDS
  __syncthreads();

  // causal / ragged-tail masking of tile j's scores, needed on few tiles
  auto need_mask = [&](int j) {
    const int k0 = k_lo + j * BK;
    return (k0 + BK > k_hi) || (CAUSAL && k0 + BK - 1 > q0w + off);
  };
  auto mask = [&](f32x16 (&s)[RB][Gm::NKB], int j) {
    const int k0 = k_lo + j * BK;
    const int ln = lane, hh = ln >> 5;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int mq = q0w + 32 * rb + (ln & 31);
#pragma unroll
      for (int kb = 0; kb < Gm::NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
          bool ok = key < k_hi;
          if (CAUSAL) ok = ok && key <= mq + off;
          if (!ok) s[rb][kb][r] = -INFINITY;
        }
    }
  };
  // weights of tile j from its scores: mask, fold the row max into the
  // reference, exp
  auto weights = [&](f32x16 (&s)[RB][Gm::NKB], int j, vec8 (&p)[RB][Gm::NKB][2]) {
    if (need_mask(j)) mask(s, j);
    const int xaddr = (lane ^ 32) << 2;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      raise_ref<D>(st[rb], tile_rowmax<Gm::NKB>(s[rb], xaddr), c);
      softmax_exp<T, D, Gm::NKB>(st[rb], s[rb], c, ref_max<D>(st[rb]), p[rb]);
    }
  };

  f32x16 sc[RB][Gm::NKB];
  vec8 pb[RB][Gm::NKB][2];  // weights of the tile whose value update is next
  if (wnt > 0) {
    qk_tile_sw<T, D, BK, RB>(sc, lds_k0, qb, lane);
    weights(sc, 0, pb);
  }
  // step 0 refills K stage 0, which every wave must have finished reading
  __syncthreads();
  // step j: K of tile j+2 and V of tile j+1 stream into the stages step
  // j-1 freed (K stage j%2, V stage (j+1)%2) while the scores of tile j+1
  // (K stage (j+1)%2) and the value update of tile j (V stage j%2) run.
  // (The stage pointers are restrict-qualified: the tile a step streams in
  // and the tiles it reads never overlap.)
  auto fill = [&](int j, uint16_t* __restrict__ kfill, uint16_t* __restrict__ vfill) {
    if (j + 2 < ntiles) dma_tile<D, BK, NT, false>(kfill, ksrc, k_lo + (j + 2) * BK, dk, tid);
    if (j + 1 < ntiles) dma_tile<D, BK, NT, true>(vfill, vsrc, k_lo + (j + 1) * BK, dv, tid);
  };
  // The scores and the value update run at raised issue priority: of the
  // two waves sharing a SIMD, the one feeding the matrix core is served
  // first and the other's vector work fills the gaps.  The step's tile
  // loads are issued after them (their issue stalls while the load queue
  // drains the other waves' tiles), then come the weights of tile j + 1.
  auto step = [&](int j, uint16_t* kf, uint16_t* vf, const uint16_t* __restrict__ kread,
                  const uint16_t* __restrict__ vread) {
    __builtin_amdgcn_s_setprio(3);
    if (j + 1 < wnt) {
      qk_tile_sw<T, D, BK, RB>(sc, kread, qb, lane);
      lds_pipeline<Gm::NKB * D / 16, RB>();
    }
    if (j < wnt) {
      pv_tile_tr<T, D, BK, RB>(st, pb, vread, lane);
      lds_pipeline_pv<D / 32 * Gm::NKB * 2, RB>();
    }
    fill(j, kf, vf);
    __builtin_amdgcn_s_setprio(0);
    if (j + 1 < wnt) weights(sc, j + 1, pb);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this step's tiles are in LDS
    __syncthreads();
  };
  for (int j = 0; j < ntiles; j += 2) {
    step(j, lds_k0, lds_v1, lds_k1, lds_v0);
    if (j + 1 < ntiles) step(j + 1, lds_k1, lds_v0, lds_k0, lds_v1);
  }

#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int oq = q0w + 32 * rb + (lane & 31);
    const bool row_ok = oq < n_q;
    const int64_t row = (q_begin + oq) * a.Hq + hq;
    if (a.s == 1) {
      // the output goes through LDS, waves 0-1 in the K stages and 2-3 in the
      // V stages (free after the last step's barrier)
      static_assert(NT == 256 && 2 * 32 * (2 * D + 16) <= 2 * TE * 2, "two waves' rows fit one stage pair");
      __attribute__((address_space(3))) char* stage =
          (__attribute__((address_space(3))) char*)(w < 2 ? lds_k : lds_v) + (w & 1) * 32 * (2 * D + 16);
      const int q0 = q0w + 32 * rb;
      uint16_t* obase = static_cast<uint16_t*>(a.o) + ((q_begin + q0) * a.Hq + hq) * D;
      float* lse = (row_ok && a.lse) ? a.lse + row : nullptr;
      row_store_staged<T, D>(st[rb], obase, int64_t(a.Hq) * D, n_q - q0, lse, stage, lane);
    } else {
      // fp16 partial rows (scaled per row) through LDS, as above
      __attribute__((address_space(3))) char* stage =
          (__attribute__((address_space(3))) char*)(w < 2 ? lds_k : lds_v) + (w & 1) * 32 * (2 * D + 16);
      const int q0 = q0w + 32 * rb;
      const int64_t prow = int64_t(si) * a.rows + row;
      uint16_t* obase = a.o_part + (int64_t(si) * a.rows + (q_begin + q0) * a.Hq + hq) * D;
      row_store_partial_staged<D>(st[rb], obase, int64_t(a.Hq) * D, n_q - q0, row_ok ? a.m_part + prow : nullptr,
                                  row_ok ? a.l_part + prow : nullptr, row_ok ? a.x_part + prow : nullptr,
                                  stage, lane);
    }
  }
}

// ---------------------------------------------------------------------------
// Block-sparse prefill.  Workgroup = 2 waves = one 64-query outer-tile row of
// one head; grid (L/64, Hq, B).  Tiles: the row's full OTs, then its part OTs.
// ---------------------------------------------------------------------------

// The part-OT predicate: x[kb][r] -> -inf where query (32*w + lane%32) of the
// OT may not attend key 32*kb + 8*(r/4) + 4*h + r%4 of the OT.
// Each element takes two vector ops: the sign-extended bit (0 or all ones)
// and a bitwise select between the score and -inf.
__device__ __forceinline__ void apply_part_mask(f32x16 (&x)[2], const uint8_t* bm, int w,
                                                int lane) {
  const int rq = 32 * w + (lane & 31);
  const int h = lane >> 5;
  const uint64_t bytes = *reinterpret_cast<const uint64_t*>(bm + rq * 8);  // [ic] for row rq
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    // bytes 4 kb .. 4 kb + 3, shifted so that nibble h of byte 4 kb + r4
    // starts at bit 8 r4
    const int wv = int(uint32_t(bytes >> (32 * kb)) >> (4 * h));
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t keep = uint32_t(__builtin_amdgcn_sbfe(wv, 8 * r4 + e, 1));
        const uint32_t xb = __float_as_uint(x[kb][4 * r4 + e]);
        x[kb][4 * r4 + e] = __uint_as_float((xb & keep) | (0xFF800000u & ~keep));
      }
  }
}

template <class T, int D>
__global__ __launch_bounds__(128, 2) void bsr_kernel(BsrArgs a) {
  constexpr int NT = 128, BK = 64, TE = BK * D;
  typedef typename T::vec8 vec8;
  // two stages of natural-layout K and V outer-tile columns, filled
  // straight from memory (attn_core.hpp), plus the part tiles' bitmaps
  __shared__ __attribute__((aligned(16))) uint16_t lds_k[2 * TE];
  __shared__ __attribute__((aligned(16))) uint16_t lds_v[2 * TE];
  __shared__ __attribute__((aligned(16))) uint8_t bm[2][512];

  int qblk, hq;
  bsr_block_head(a.num_blocks, a.Hq, qblk, hq);
  const int b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
  const int g = hq / a.G;
  const int mrow = (hq / a.heads_per_mask) * (a.num_blocks + 1) + qblk;  // this head's mask
  const int f0 = a.full_indptr[mrow], n_full = a.full_indptr[mrow + 1] - f0;
  const int p0 = a.part_indptr[mrow], n_part = a.part_indptr[mrow + 1] - p0;
  const int ntiles = n_full + n_part;

  const int64_t L = a.L;
  const int my_q = qblk * 64 + 32 * w + (lane & 31);
  const uint16_t* Q = static_cast<const uint16_t*>(a.q);
  u32x4 qb[1][D / 16];
  load_q<D>(qb[0], Q + ((int64_t(b) * L + my_q) * a.Hq + hq) * D, lane);

  RowState<D> st[1];
  row_state_init(st[0]);

  const int row_stride = a.Hkv * D;
  const uint16_t* kbase = static_cast<const uint16_t*>(a.k) + int64_t(b) * L * row_stride + int64_t(g) * D;
  const uint16_t* vbase = static_cast<const uint16_t*>(a.v) + int64_t(b) * L * row_stride + int64_t(g) * D;
  const DmaSrc ksrc = dma_src(kbase, row_stride, int(L)), vsrc = dma_src(vbase, row_stride, int(L));
  const DmaLane<D, BK, NT, false> dk(row_stride, tid);
  const DmaLane<D, BK, NT, true> dv(row_stride, tid);

  // the key block of stored tile j (full tiles first, then part tiles) into
  // the given stage, and its bitmap word if it is a part tile
  uint64_t word = 0;
  auto fetch = [&](int j, uint16_t* kd, uint16_t* vd) {
    const bool part = j >= n_full;
    const int kblk = part ? a.part_kblock[p0 + j - n_full] : a.full_kblock[f0 + j];
    if (part && tid < 64) word = a.part_bits[int64_t(p0 + j - n_full) * 64 + tid];
    dma_tile<D, BK, NT, false>(kd, ksrc, kblk * 64, dk, tid);
    dma_tile<D, BK, NT, true>(vd, vsrc, kblk * 64, dv, tid);
  };
  if (ntiles > 0) fetch(0, lds_k, lds_v);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): tile 0 is in LDS
  if (ntiles > 0 && n_full == 0) bitmap_store(word, bm[0], tid);
  __syncthreads();
  for (int j = 0; j < ntiles; ++j) {
    const int cur = j & 1, nxt = cur ^ 1;
    // tile j + 1 streams into the stage tile j - 1 released
    if (j + 1 < ntiles) fetch(j + 1, lds_k + nxt * TE, lds_v + nxt * TE);
    f32x16 s[1][2];
    vec8 pb[1][2][2];
    __builtin_amdgcn_s_setprio(3);
    qk_tile_sw<T, D, BK, 1>(s, lds_k + cur * TE, qb, lane);
    __builtin_amdgcn_s_setprio(0);
    if (j >= n_full) apply_part_mask(s[0], bm[cur], w, lane);
    const float mref = softmax_max<D, 2>(st[0], s[0], a.scale_log2, 0);
    softmax_exp<T, D, 2>(st[0], s[0], a.scale_log2, mref, pb[0]);
    __builtin_amdgcn_s_setprio(3);
    pv_tile_tr<T, D, BK, 1>(st, pb, lds_v + cur * TE, lane);
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): tile j + 1 (and its word) arrived
    if (j + 1 < ntiles && j + 1 >= n_full) bitmap_store(word, bm[nxt], tid);
    __syncthreads();
  }

  // the output goes through the free K stages (attn_core.hpp, row_store_staged)
  static_assert(NT == 128 && 2 * 32 * (2 * D + 16) <= 2 * TE * 2, "the waves' rows fit the K stages");
  const int64_t orow_idx = (int64_t(b) * L + my_q) * a.Hq + hq;
  uint16_t* obase = static_cast<uint16_t*>(a.o) + ((int64_t(b) * L + qblk * 64 + 32 * w) * a.Hq + hq) * D;
  row_store_staged<T, D>(st[0], obase, int64_t(a.Hq) * D, 32, a.lse ? a.lse + orow_idx : nullptr,
                         (__attribute__((address_space(3))) char*)lds_k + w * 32 * (2 * D + 16), lane);
}

// The D = 64 form: two halves of a row's stored tiles in one workgroup.
// Wave w takes query rows 32 (w % 2) .. +31 of the block row and the tiles
// of half kh = w / 2 of the row's list (full tiles, then part tiles, cut
// at ceil(n / 2)), each half with its own one-stage K/V and bitmap slot
// (a half waits for each of its tiles); after the last tile the second
// half's (O, m, l) meet the first's in LDS and combine with log-sum-exp
// weights.  At 17 KB per half and 120 registers, four such workgroups
// share a compute unit: four waves per SIMD hide each other's waits, and
// a row's tiles take half as long (C5: 122 -> 109 us against the
// two-stage two-wave form; key-column tiles of 8192 keys 575 -> 393 us).
template <class T>
__global__ __launch_bounds__(256, 4) void bsr_kernel_halves(BsrArgs a) {
  constexpr int D = 64, NT = 128, BK = 64, TE = BK * D;
  typedef typename T::vec8 vec8;
  __shared__ __attribute__((aligned(16))) uint16_t lds_k[2 * TE];
  __shared__ __attribute__((aligned(16))) uint16_t lds_v[2 * TE];
  __shared__ __attribute__((aligned(16))) uint8_t bm[2][512];

  int qblk, hq;
  bsr_block_head(a.num_blocks, a.Hq, qblk, hq);
  const int b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rw = w & 1, kh = w >> 1, htid = tid & 127;  // row half, tile half, thread in half
  const int g = hq / a.G;
  const int mrow = (hq / a.heads_per_mask) * (a.num_blocks + 1) + qblk;
  const int f0 = a.full_indptr[mrow], n_full = a.full_indptr[mrow + 1] - f0;
  const int p0 = a.part_indptr[mrow], n_part = a.part_indptr[mrow + 1] - p0;
  const int ntiles = n_full + n_part;
  const int nh = (ntiles + 1) / 2;                     // steps: tiles of the longer half
  const int j0 = kh * nh, j1 = kh ? ntiles : nh;       // this half's tiles [j0, j1)

  const int64_t L = a.L;
  const int my_q = qblk * 64 + 32 * rw + (lane & 31);
  const uint16_t* Q = static_cast<const uint16_t*>(a.q);
  u32x4 qb[1][D / 16];
  load_q<D>(qb[0], Q + ((int64_t(b) * L + my_q) * a.Hq + hq) * D, lane);
  RowState<D> st[1];
  row_state_init(st[0]);

  const int row_stride = a.Hkv * D;
  const uint16_t* kbase = static_cast<const uint16_t*>(a.k) + int64_t(b) * L * row_stride + int64_t(g) * D;
  const uint16_t* vbase = static_cast<const uint16_t*>(a.v) + int64_t(b) * L * row_stride + int64_t(g) * D;
  const DmaSrc ksrc = dma_src(kbase, row_stride, int(L)), vsrc = dma_src(vbase, row_stride, int(L));
  const DmaLane<D, BK, NT, false> dk(row_stride, htid);
  const DmaLane<D, BK, NT, true> dv(row_stride, htid);
  uint16_t* const kst = lds_k + kh * TE;
  uint16_t* const vst = lds_v + kh * TE;
  uint8_t* const bmh = bm[kh];

  // tile j of the row into this half's slot (its two waves load it), with
  // its bitmap word if it is a part tile (lanes of the half's first wave)
  uint64_t word = 0;
  auto fetch = [&](int j) {
    const bool part = j >= n_full;
    const int kblk = part ? a.part_kblock[p0 + j - n_full] : a.full_kblock[f0 + j];
    if (part && htid < 64) word = a.part_bits[int64_t(p0 + j - n_full) * 64 + htid];
    dma_tile<D, BK, NT, false>(kst, ksrc, kblk * 64, dk, htid);
    dma_tile<D, BK, NT, true>(vst, vsrc, kblk * 64, dv, htid);
  };
  if (j0 < j1) fetch(j0);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  if (j0 < j1 && j0 >= n_full) bitmap_store(word, bmh, htid);
  __syncthreads();
  for (int t = 0; t < nh; ++t) {
    const int j = j0 + t;
    if (j < j1) {
      f32x16 s[1][2];
      vec8 pb[1][2][2];
      __builtin_amdgcn_s_setprio(3);
      qk_tile_sw<T, D, BK, 1>(s, kst, qb, lane);
      __builtin_amdgcn_s_setprio(0);
      if (j >= n_full) apply_part_mask(s[0], bmh, rw, lane);
      const float mref = softmax_max<D, 2>(st[0], s[0], a.scale_log2, 0);
      softmax_exp<T, D, 2>(st[0], s[0], a.scale_log2, mref, pb[0]);
      __builtin_amdgcn_s_setprio(3);
      pv_tile_tr<T, D, BK, 1>(st, pb, vst, lane);
      __builtin_amdgcn_s_setprio(0);
    }
    __syncthreads();  // both halves are done with their slots
    if (j + 1 < j1) fetch(j + 1);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    if (j + 1 < j1 && j + 1 >= n_full) bitmap_store(word, bmh, htid);
    __syncthreads();
  }

  // second half -> LDS, reusing the slots: O^T in the K slots (2 waves x
  // D / 2 floats x 64 lanes = 16 KB, float r of lane l at r * 64 + l), m
  // and l in the V slots
  float* xo = reinterpret_cast<float*>(lds_k) + rw * (D / 2) * 64 + lane;
  float* xm = reinterpret_cast<float*>(lds_v) + rw * 128 + lane;
  if (kh == 1) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) xo[(16 * db + r) * 64] = st[0].o[db][r];
    xm[0] = st[0].m;
    xm[64] = st[0].l;
  }
  __syncthreads();
  if (kh == 1) return;
  {
    const float* p = xo;
    const float m2 = xm[0], l2 = xm[64];
    const float m1 = st[0].m;
    const float M = fmaxf(m1, m2);
    // m = -inf marks a half with no valid key so far: weight 0
    const float a1 = m1 == -INFINITY ? 0.f : fexp2(m1 - M);
    const float a2 = m2 == -INFINITY ? 0.f : fexp2(m2 - M);
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) st[0].o[db][r] = st[0].o[db][r] * a1 + p[(16 * db + r) * 64] * a2;
    st[0].l = st[0].l * a1 + l2 * a2;
    st[0].m = M;
  }
  // the output goes through the V slots past the (m, l) exchange (attn_core.hpp,
  // row_store_staged)
  static_assert(1024 + 2 * 32 * (2 * D + 16) <= 2 * TE * 2, "the waves' rows fit the V slots");
  const int64_t orow_idx = (int64_t(b) * L + my_q) * a.Hq + hq;
  uint16_t* obase = static_cast<uint16_t*>(a.o) + ((int64_t(b) * L + qblk * 64 + 32 * rw) * a.Hq + hq) * D;
  row_store_staged<T, D>(st[0], obase, int64_t(a.Hq) * D, 32, a.lse ? a.lse + orow_idx : nullptr,
                         (__attribute__((address_space(3))) char*)lds_v + 1024 + rw * 32 * (2 * D + 16), lane);
}

// Dense expansion of the two-level mask with the kernel's own predicate:
// workgroup = 2 waves = one query block row, lanes laid out as in bsr_kernel.
__global__ __launch_bounds__(128) void bsr_decode_kernel(const int32_t* full_indptr,
                                                         const int32_t* full_kblock,
                                                         const int32_t* part_indptr,
                                                         const int32_t* part_kblock,
                                                         const uint64_t* part_bits, int nblk,
                                                         uint8_t* dense) {
  __shared__ __attribute__((aligned(16))) uint8_t bm[512];
  const int qblk = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5;
  const int64_t L = int64_t(nblk) * 64;
  const int my_q = qblk * 64 + 32 * w + (lane & 31);
  uint8_t* drow = dense + my_q * L;
  for (int64_t e = tid; e < 64 * L; e += 128) dense[int64_t(qblk) * 64 * L + e] = 0;
  __syncthreads();
  for (int j = full_indptr[qblk]; j < full_indptr[qblk + 1]; ++j) {
    const int kb0 = full_kblock[j] * 64;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) drow[kb0 + 32 * kb + 8 * (r >> 2) + 4 * h + (r & 3)] = 1;
  }
  for (int j = part_indptr[qblk]; j < part_indptr[qblk + 1]; ++j) {
    __syncthreads();
    bitmap_store(tid < 64 ? part_bits[int64_t(j) * 64 + tid] : 0, bm, tid);
    __syncthreads();
    f32x16 x[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) x[kb][r] = 0.f;
    apply_part_mask(x, bm, w, lane);
    const int kb0 = part_kblock[j] * 64;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        drow[kb0 + 32 * kb + 8 * (r >> 2) + 4 * h + (r & 3)] = x[kb][r] == 0.f ? 1 : 0;
  }
}

// ---- launchers -------------------------------------------------------------

template <class T, int D>
static void launch_prefill_t(const PrefillArgs& a, hipStream_t st) {
  constexpr int BQ = kPrefillBQ;
  const dim3 grid(a.Hq, a.B, unsigned((a.max_q_len + BQ - 1) / BQ * a.s));
  const dim3 block(64 * kPrefillWaves);
  if (a.causal) hipLaunchKernelGGL((prefill_kernel<T, D, true>), grid, block, 0, st, a);
  else hipLaunchKernelGGL((prefill_kernel<T, D, false>), grid, block, 0, st, a);
}

int prefill_rows_per_workgroup() { return kPrefillBQ; }

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t st) {
  if (a.max_q_len <= 0) return hipSuccess;
  if (a.dtype == 1) {
    if (a.D == 64) launch_prefill_t<BF16, 64>(a, st); else launch_prefill_t<BF16, 128>(a, st);
  } else {
    if (a.D == 64) launch_prefill_t<F16, 64>(a, st); else launch_prefill_t<F16, 128>(a, st);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.s == 1) return e;
  // split partials -> o / lse by log-sum-exp weights (the standalone merge,
  // as attn_merge_lse)
  MergeArgs m{nullptr, a.m_part, a.l_part, a.s, int(a.rows), a.D, a.o, a.dtype, a.lse, a.o_part, a.x_part};
  return launch_merge(m, st);
}

hipError_t launch_prefill_bsr(const BsrArgs& a, hipStream_t st) {
  const dim3 grid(a.num_blocks, a.Hq, a.B);
  if (a.D == 64) {  // two-halves form
    if (a.dtype == 1) hipLaunchKernelGGL((bsr_kernel_halves<BF16>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((bsr_kernel_halves<F16>), grid, dim3(256), 0, st, a);
  } else {
    if (a.dtype == 1) hipLaunchKernelGGL((bsr_kernel<BF16, 128>), grid, dim3(128), 0, st, a);
    else hipLaunchKernelGGL((bsr_kernel<F16, 128>), grid, dim3(128), 0, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_bsr_decode(const int32_t* full_indptr, const int32_t* full_kblock,
                             const int32_t* part_indptr, const int32_t* part_kblock,
                             const uint64_t* part_bits, int num_blocks, uint8_t* dense,
                             hipStream_t st) {
  hipLaunchKernelGGL(bsr_decode_kernel, dim3(num_blocks), dim3(128), 0, st, full_indptr,
                     full_kblock, part_indptr, part_kblock, part_bits, num_blocks, dense);
  return hipGetLastError();
}

}  // namespace rattn
