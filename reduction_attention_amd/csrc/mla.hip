// mla.hip -- multi-head latent attention (MLA) decode on gfx950, absorbed form.
//
// The Cleave arXiv abstract lists MLA among the attention subgraphs the
// method handles.  In its absorbed decode form every query head attends to
// one shared cache row per token: a latent vector of Dc = 512 elements
// followed by a rotary key part of Dr = 64, 576 elements in all.  The score
// of head h against token j is scale * q_h . row_j over all 576 elements;
// the output of head h is the softmax-weighted sum of the latent parts
// (the first 512 elements) of the rows.  So K is the whole row and V is its
// first 512 elements: the same bytes, read once for both.
//
// Decomposition: the Split operator cuts each request's keys into chunks of
// c = ceil(max_kv_len / s) (Cleave article on tip.co.jp, "Split演算子による
// Split-Kの対応"), one workgroup per (16 query heads, chunk, request) -- or
// per 64 heads when the head count is a multiple of 64 (mla_wide_kernel,
// below, whose chunks are packed so that only the chunks a request has are
// launched); the partials are merged with log-sum-exp weights by
// mla_merge_kernel (end of this file).
// Inside a chunk, 32-key tiles of cache rows are staged in LDS and each tile
// feeds the score, the online max/sum and the value update in one pass
// ("複数リダクションのスケジューリング": iterative tiling, horizontal fusion).
//
// Workgroup = W waves (4 by default; two workgroups share a compute unit,
// so one's barriers and LDS latencies overlap the other's work).  The
// scores of a 32-key tile for the 16 heads (S^T = K Q^T on 16x16x32 MFMAs,
// K from LDS) are split W ways: wave w takes the 16 keys 16 * (w / (W/2))
// .. and a 1 / (W/2) share of the 576 dims, and the partial sums meet in
// LDS; every wave then adds the same partials in the same order, runs the
// same online softmax, and updates its 512 / W output dims (O^T += V^T
// P^T, V^T from transposing LDS reads).
#include "device.hpp"
#include "launch.hpp"
#include <type_traits>

namespace rattn {

typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kMlaDc = 512, kMlaDr = 64, kMlaD = kMlaDc + kMlaDr;  // cache row: 576 elements
constexpr int kMlaBK = 32;                      // keys per tile
constexpr int kMlaChunks = kMlaD / 8;           // 16-byte chunks per cache row (72)
constexpr int kMlaLdsRow = kMlaChunks + 1;      // LDS row: one pad chunk (rows 36 banks apart)
constexpr int kMlaWaves = 4;
constexpr int kMlaThreads = 64 * kMlaWaves;
// A tile goes from HBM straight into an LDS stage: 64-lane x 16-byte load
// instructions, each filling 1 KB of the stage (37 per tile, the last one
// partly padding), kMlaStages stages in a ring (2 by default: 80 KB with
// the score exchange, two workgroups per compute unit).
constexpr int kMlaInstr = (kMlaBK * kMlaLdsRow + 63) / 64;  // 37
constexpr int kMlaPerWave = (kMlaInstr + kMlaWaves - 1) / kMlaWaves;  // loads per wave and tile (at most)
constexpr int kMlaStageBytes = kMlaInstr * 1024;
constexpr int kMlaStage = kMlaStageBytes / 2;  // 16-bit elements per stage
constexpr int kMlaStages = 2;
// s_waitcnt vmcnt(n) (gfx9 encoding: vmcnt bits 3:0 and 15:14; expcnt and
// lgkmcnt fields at their no-wait maximum) that lets the loads of all
// stages but two stay in flight: the tile the next step reads has arrived
// (waves that issue one load more per tile only wait a little earlier)
constexpr int kVmAhead = (kMlaStages - 2) * (kMlaInstr / kMlaWaves);
constexpr int kVmcntNext = 0x0F70 | (kVmAhead & 15) | ((kVmAhead >> 4) << 14);

// Work unit of workgroup L of the 1-D grid.  Workgroups are dealt to the
// eight XCDs round robin by linear index and each XCD has its own L2, so
// the head groups of one (chunk, request) unit are given consecutive
// indices on the same XCD: unit = 8 * (r / HG) + L % 8, head group r % HG,
// r = L / 8.  Returns false for the padding past the last unit.
__device__ __forceinline__ bool mla_unit(int L, int HG, int units, int& hg, int& unit) {
  const int r = L >> 3;
  hg = r % HG;
  unit = (r / HG) * 8 + (L & 7);
  return unit < units;
}

// Chunk plan of the many-head kernel on ragged batches, packed: request b
// owns n_b = min(ceil(len_b / c), s)
// consecutive units (one for an empty request, which writes its zero rows),
// so no workgroup slot goes to a split the request does not have and the
// units dealt to each XCD carry nearly equal work.  The request of a unit is
// found by a prefix sum of n_b over the requests, 64 at a time across the
// lanes (the result is uniform over the wave).  Returns false past the last
// unit.
__device__ __forceinline__ bool mla_packed_unit(const MlaArgs& a, int unit, int lane, int& b, int& i) {
  const int64_t c = a.chunk;
  b = -1;
  i = 0;
  int base = 0;  // units owned by the requests before j0 (at most s * B < 2^27)
  for (int j0 = 0; j0 < a.B; j0 += 64) {
    const int j = j0 + lane;
    int nb = 0;
    if (j < a.B) {
      const int64_t len = int64_t(a.kv_indptr[j + 1]) - a.kv_indptr[j];
      nb = len > 0 ? int(min((len + c - 1) / c, int64_t(a.s))) : 1;
    }
    int incl = nb;  // inclusive prefix sum across the lanes
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int t = __shfl_up(incl, d);
      if (lane >= d) incl += t;
    }
    const int first = base + incl - nb;
    const uint64_t hit = __ballot(nb > 0 && unit >= first && unit < first + nb);
    if (hit) {
      const int l = __ffsll((unsigned long long)hit) - 1;
      b = __builtin_amdgcn_readfirstlane(j0 + l);
      i = __builtin_amdgcn_readfirstlane(unit - __shfl(first, l));
      return true;
    }
    base += __shfl(incl, 63);
  }
  return false;
}

// Transposing LDS read (ds_read_b64_tr_b16) at a byte offset from base: see
// the lane layout at its use below.
__device__ __forceinline__ u32x2 mla_tr_read(const uint16_t* base, int byte_off) {
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  const char* p = reinterpret_cast<const char*>(base) + byte_off;
  const v4i16 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(p));
  return __builtin_bit_cast(u32x2, x);
}

// Split partials are kept in fp16 with each 128-dim quarter of a row divided
// by a power of two 2^e, e the binary exponent of the quarter's largest
// magnitude: every stored value then lies within [-1, 1], where fp16 keeps
// 11 significant bits, so a stored element is off by at most 2^-12 of the
// quarter's largest value (a bf16 copy would be off by up to 2^-9 of the
// element), and neither the inputs' range nor fp16's can overflow it.
// Dividing by a power of two is exact; the scale 2^e goes to x_part.
__device__ __forceinline__ int mla_part_exp(float amax) {
  const int e = __builtin_amdgcn_frexp_expf(amax);
  return e < -126 ? -126 : (e > 127 ? 127 : e);
}

template <class T>
__global__ __launch_bounds__(kMlaThreads, 8 / kMlaWaves) void mla_decode_kernel(MlaArgs a) {
  typedef typename T::vec8 vec8;
  __shared__ __attribute__((aligned(16))) uint16_t lds[kMlaStages * kMlaStage];
  const int HG = (a.H + 15) / 16;
  int hg, unit;
  if (!mla_unit(blockIdx.x, HG, a.s * a.B, hg, unit)) return;
  const int b = unit / a.s, i = unit % a.s;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c16 = lane & 15, h4 = lane >> 4;
  const int H = a.H;
  const int64_t rows = int64_t(a.B) * H;
  const int64_t kb0 = a.kv_indptr[b], kb1 = a.kv_indptr[b + 1];
  const int n_b = int(kb1 - kb0);
  const int lo = int(int64_t(i) * a.chunk < n_b ? int64_t(i) * a.chunk : n_b);
  const int hi = lo + a.chunk < n_b ? lo + a.chunk : n_b;
  const int64_t row0 = int64_t(b) * H + 16 * hg;  // this workgroup's first query head row
  const int nh = H - 16 * hg < 16 ? H - 16 * hg : 16;  // heads in this group
  const int splits_b = min((n_b + a.chunk - 1) / a.chunk, a.s);  // s bounds the slots
  if (lo >= hi) {  // split unused by this request
    if (i == 0) {  // empty request: O = 0, LSE = -inf
      typename T::elem* o = static_cast<typename T::elem*>(a.o) + row0 * kMlaDc;
      for (int e = tid; e < nh * kMlaDc; e += kMlaThreads) o[e] = typename T::elem(0.f);
      if (a.lse && tid < nh) a.lse[row0 + tid] = -INFINITY;
    }
    return;
  }
  const int n = hi - lo;
  const int ntiles = (n + kMlaBK - 1) / kMlaBK;

  // The wave's share of the scores: key tile kt = w / (W/2) (keys 16 kt ..
  // 16 kt + 15 of each 32-key tile), slabs u0 .. u0 + ns - 1 of the 18
  // (dims 32 u0 ..; W = 4: halves of 9 slabs, W = 8: 4, 5, 4, 5).  Q^T
  // operand: head c16 of the group (zero past the last head), slab u0 + u
  // -> dims 32 (u0 + u) + 8 h4 .. +8.
  constexpr int DQ = kMlaWaves / 2;             // parts of the dims
  constexpr int NS = (kMlaD / 32 + DQ - 1) / DQ;  // slabs of the larger parts
  const int kt = w / DQ, dq = w % DQ;
  const int u0 = (kMlaD / 32) * dq / DQ, ns = (kMlaD / 32) * (dq + 1) / DQ - u0;
  u32x4 qb[NS];  // loaded at start-up, after tile 0's loads are issued
  // partial score tiles of the waves: sx[w][lane] = lane's four
  // scores (head c16, keys 16 kt + 4 h4 + r) over the wave's slabs
  __shared__ __attribute__((aligned(16))) f32x4 sx[kMlaWaves][64];

  // Direct-to-LDS tile loads.  Instruction x (wave x % 8 issues it) fills
  // stage chunks 64x .. 64x + 63; lane l's chunk q = 64x + l is row q / 73,
  // slot q % 73 of the padded stage, fetched from chunk 72 * row + slot of
  // the tile's rows; the pad slot 72 and chunks past the 32 rows fetch
  // from an offset outside every resource and receive zeros.  The offsets
  // are the same for every tile, so they are computed once.  A tile's
  // resource ends at the chunk's last key: keys past it arrive as zeros
  // (their scores are masked, and zero values add nothing); a tile wholly
  // past it reads no memory.
  const int nwi = __builtin_amdgcn_readfirstlane((kMlaInstr - w + kMlaWaves - 1) / kMlaWaves);
  int voff[kMlaPerWave];
#pragma unroll
  for (int k = 0; k < kMlaPerWave; ++k) {
    const int q = 64 * (w + kMlaWaves * k) + lane;
    const int r = q / kMlaLdsRow, c = q % kMlaLdsRow;
    voff[k] = (c < kMlaChunks && r < kMlaBK) ? (r * kMlaChunks + c) * 16 : 0x40000000;
  }
  typedef int i32x4 __attribute__((ext_vector_type(4)));
  const uint64_t cbase = uint64_t(size_t(static_cast<const uint16_t*>(a.kv) + (kb0 + lo) * kMlaD));
  const uint32_t lds0 = uint32_t(size_t((__attribute__((address_space(3))) uint16_t*)lds)) + w * 1024;
  auto dma = [&](int tile) {
    const int key0 = tile * kMlaBK;
    int left = n - key0;
    left = left < 0 ? 0 : (left > kMlaBK ? kMlaBK : left);
    const uint64_t addr = cbase + uint64_t(uint32_t(key0)) * (2 * kMlaD);
    const i32x4 rsv = {__builtin_amdgcn_readfirstlane(int(uint32_t(addr))),
                       __builtin_amdgcn_readfirstlane(int(uint32_t(addr >> 32) & 0xffffu)),
                       __builtin_amdgcn_readfirstlane(left * 2 * kMlaD), 0x00020000};
    const uint32_t st = lds0 + uint32_t(tile % kMlaStages) * kMlaStageBytes;
#pragma unroll
    for (int k = 0; k < kMlaPerWave; ++k)
      if (k < nwi)
        __asm__ volatile(
            "s_mov_b32 m0, %0\n\t"
            "buffer_load_dwordx4 %1, %2, 0 offen lds"
            :
            : "s"(__builtin_amdgcn_readfirstlane(st + k * 1024 * kMlaWaves)), "v"(voff[k]), "s"(rsv)
            : "memory", "m0");
  };

  // running state of head c16: m (log2 units, same in the four h4 lanes),
  // this lane's share of the sum, O^T accumulators of the wave's 512 / W
  // dims: o[blk][r] = dim (512 / W) w + 16 blk + 4 h4 + r
  constexpr int NB = kMlaDc / 16 / kMlaWaves;  // 16-dim blocks per wave
  float m = -INFINITY, l = 0.f;
  f32x4 o[NB];
#pragma unroll
  for (int k = 0; k < NB; ++k) o[k] = f32x4{0.f, 0.f, 0.f, 0.f};

  // transposing-read addresses (bytes, within a stage): lane q + 4e of its
  // 16-lane group points at row k0 + e, dims dbase + 4q; the group h4 reads
  // rows 4*h4 + e (keys of its P slots 0..3) and 16 + 4*h4 + e (slots 4..7)
  const int tq = lane & 3, te = (lane >> 2) & 3;
  const int tr0 = 2 * ((4 * h4 + te) * kMlaLdsRow * 8 + 16 * NB * w + 4 * tq);
  const int tr1 = tr0 + 2 * 16 * kMlaLdsRow * 8;

  // Step j: the load of tile j + S - 1 (S stages) goes into the stage tile
  // j - 1 used (free since the barrier that ended step j - 1), tile j is
  // computed, and the step ends once tile j + 1 is in LDS: each wave waits
  // for its own loads of it, then the barrier publishes them.  Tiles past the chunk are issued too (they
  // read nothing), so the count of loads in flight never depends on the
  // path.
  auto step = [&](int j) {
    dma(j + kMlaStages - 1);
    const uint16_t* cur = lds + (j % kMlaStages) * kMlaStage;
    // this wave's partial S^T tile (16 keys x 16 heads: lane (c16, h4) gets
    // head c16, keys 16 kt + 4 h4 + r), operands read from LDS in one batch
    {
      const uint16_t* kp = cur + ((16 * kt + c16) * kMlaLdsRow + 4 * u0 + h4) * 8;
      u32x4 ka[NS];
#pragma unroll
      for (int u = 0; u < NS; ++u)
        if (u < ns) ka[u] = *reinterpret_cast<const u32x4*>(kp + 32 * u);
      f32x4 sp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < NS; ++u)
        if (u < ns) sp = T::mfma16(as<vec8>(ka[u]), as<vec8>(qb[u]), sp);
      sx[w][lane] = sp;
    }
    __syncthreads();
    // the whole tile's scores, summed the same way in every wave
    f32x4 s[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      s[t] = sx[DQ * t][lane];
#pragma unroll
      for (int q = 1; q < DQ; ++q) s[t] += sx[DQ * t + q][lane];
    }
    float x[8];
    const int key0 = j * kMlaBK;
    const bool tail = key0 + kMlaBK > n;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float y = s[t][r] * a.scale_log2;
        if (tail && key0 + 16 * t + 4 * h4 + r >= n) y = -INFINITY;
        x[4 * t + r] = y;
      }
    float mx = max3(x[0], x[1], max3(x[2], x[3], max3(x[4], x[5], fmaxf(x[6], x[7]))));
    mx = fmaxf(mx, shfl_xor(mx, 16));
    mx = fmaxf(mx, shfl_xor(mx, 32));
    // every tile holds at least one valid key, so mx and m_new are finite
    const float m_new = fmaxf(m, mx);
    const float alpha = fexp2(m - m_new);
    m = m_new;
    f32x8 p;
    float psum = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      p[k] = fexp2(x[k] - m_new);
      psum += p[k];
    }
    l = l * alpha + psum;
    const vec8 pb = T::cvt8(p);
    u32x2 v0[NB], v1[NB];
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
      v0[blk] = mla_tr_read(cur, tr0 + 32 * blk);
      v1[blk] = mla_tr_read(cur, tr1 + 32 * blk);
    }
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
      const u32x4 av = {v0[blk][0], v0[blk][1], v1[blk][0], v1[blk][1]};
      o[blk] *= alpha;
      o[blk] = T::mfma16(as<vec8>(av), pb, o[blk]);
    }
    __builtin_amdgcn_s_waitcnt(kVmcntNext);  // tile j + 1 has arrived
    __syncthreads();
  };
  // Start-up: tile 0 and the query operand come in together (the wait
  // for the query below also covers tile 0, issued before it), then the
  // tiles of the other stages but one are issued.
  dma(0);
  {
    const bool ok = c16 < nh;
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + (row0 + (ok ? c16 : 0)) * kMlaD +
                         32 * u0 + 8 * h4;
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      qb[u] = (ok && u < ns) ? ldg128(qp + 32 * u) : u32x4{0u, 0u, 0u, 0u};
    }
    // consume the loads now: the tile loads below are invisible to the
    // compiler's wait counting, so no later wait may be left to it
#pragma unroll
    for (int u = 0; u < NS; ++u) __asm__ volatile("" ::"v"(qb[u]));
  }
#pragma unroll
  for (int t = 1; t < kMlaStages - 1; ++t) dma(t);
  __syncthreads();
  for (int j = 0; j < ntiles; ++j) step(j);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): no load outlives the workgroup

  // head sums over the four h4 lanes; lane (c16, h4) writes dims
  // (512 / W) w + 16blk + 4h4 .. +4 of head c16
  l += shfl_xor(l, 16);
  l += shfl_xor(l, 32);
  if (c16 >= nh) return;
  const int64_t row = row0 + c16;
  const float inv = 1.f / l;
  if (splits_b == 1) {
    typename T::elem* orow = static_cast<typename T::elem*>(a.o) + row * kMlaDc + 16 * NB * w + 4 * h4;
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
      f32x8 y;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        y[r] = o[blk][r] * inv;
        y[4 + r] = 0.f;
      }
      const u32x4 bits = __builtin_bit_cast(u32x4, T::cvt8(y));
      *reinterpret_cast<u32x2*>(orow + 16 * blk) = u32x2{bits[0], bits[1]};
    }
    if (a.lse && w == 0 && h4 == 0) a.lse[row] = (m + flog2(l)) * kLn2;
  } else {
    // the wave's dims are quarter w of the row (lanes c16 + 16 h4 hold them)
    static_assert(16 * NB == 128, "one wave per 128-dim quarter");
    float amax = 0.f;
#pragma unroll
    for (int blk = 0; blk < NB; ++blk)
#pragma unroll
      for (int r = 0; r < 4; ++r) amax = fmaxf(amax, fabsf(o[blk][r]));
    amax = fmaxf(amax, shfl_xor(amax, 16));
    amax = fmaxf(amax, shfl_xor(amax, 32));
    const int e = mla_part_exp(amax * inv);
    uint16_t* prow = a.o_part + (int64_t(i) * rows + row) * kMlaDc + 16 * NB * w + 4 * h4;
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
      f32x8 y;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        y[r] = __builtin_amdgcn_ldexpf(o[blk][r] * inv, -e);
        y[4 + r] = 0.f;
      }
      const u32x4 bits = __builtin_bit_cast(u32x4, F16::cvt8(y));
      *reinterpret_cast<u32x2*>(prow + 16 * blk) = u32x2{bits[0], bits[1]};
    }
    if (h4 == 0) a.x_part[(int64_t(i) * rows + row) * 4 + w] = __builtin_amdgcn_ldexpf(1.f, e);
    if (w == 0 && h4 == 0) {
      a.m_part[int64_t(i) * rows + row] = m * kLn2;
      a.l_part[int64_t(i) * rows + row] = l;
    }
  }
}

// ---------------------------------------------------------------------------
// Many heads (H a multiple of 64): the heads are the rows of the score
// matrix, so the tile feeds 32x32x16 MFMAs with K and V from LDS as in
// prefill.  Workgroup = 4 waves over 64 heads of one (chunk, request), one
// wave per SIMD: wave w takes head block hb = w / 2 (32 heads) and half
// dh = w % 2 of the dims -- dims 288 dh .. 288 dh + 287 of the score
// contraction (eighteen 16-dim steps) and output dims 256 dh .. 256 dh +
// 255.  The two waves of a head block swap their partial scores through
// LDS once per tile; each adds the pair in the same order (half 0 + half
// 1), so both hold the same full scores, run the same online softmax and
// feed the same weights to their own output half: no weight crosses
// waves.
//
// Schedule (two barriers per tile): step j turns tile j's swapped partial
// scores into weights, issues the load of tile j + 3 and computes tile
// j + 1's partial scores; a barrier then marks that every wave has read
// its partner's partials of tile j, so the one exchange buffer takes tile
// j + 1's; the step runs tile j's value update, waits for tile j + 2's
// loads and meets the other waves.  LDS holds four stages (tile j: values,
// tile j + 1: keys, tiles j + 2 and j + 3: streaming in, so a tile's loads
// have two steps to arrive; timing copies without the loads ran a third
// faster) and one tile's partial scores: 160 KB.
//
// Softmax reference: the row max of the chunk's first tile, kept for the
// whole chunk, so the value accumulators are never rescaled.  A later
// weight above 2^64 (2^15 for fp16 operands) sets a flag; the workgroup
// then runs the chunk again against the chunk's true row max (found on the
// first pass), which no score exceeds.  Keys far below the reference only
// lose weights that are negligible against the reference key's weight of 1.
//
// LDS rows: 72 chunks of 16 bytes per cache row with the chunk index XOR-ed
// by f(row) = 2 (row % 4) + (row / 4) % 2, so that both the 16-byte K reads
// (eight consecutive rows, one chunk) and the transposing V reads (four
// consecutive rows, two chunks) hit distinct banks.  A tile arrives through
// 36 direct-to-LDS load instructions of 1 KB, x = w + 4 k.
// ---------------------------------------------------------------------------
constexpr int kMwBK = 32;
constexpr int kMwInstr = kMwBK * kMlaChunks / 64;  // 36 load instructions of 1 KB per tile
constexpr int kMwWaves = 4;
constexpr int kMwPerWave = kMwInstr / kMwWaves;    // 9
constexpr int kMwStageBytes = kMwInstr * 1024;     // 36,864
constexpr int kMwStages = 4;
constexpr int kMwOutRow = 528;  // LDS bytes per head row of the output staging
static_assert(kMwInstr % kMwWaves == 0, "every wave issues the same loads");
static_assert(kMwWaves * 32 * kMwOutRow <= kMwStages * kMwStageBytes, "output staging fits the stages");
// A weight above 2^mw_overflow forces the exact pass: 2^64 for bf16 (its
// range is fp32's, and sums of such weights stay far from overflow), 2^15
// for fp16, whose largest finite value is just below 2^16.
__device__ __forceinline__ constexpr float mw_overflow(BF16) { return 64.f; }
__device__ __forceinline__ constexpr float mw_overflow(F16) { return 15.f; }

__device__ __forceinline__ int mw_swz(int row) { return ((row & 3) << 1) | ((row >> 2) & 1); }

// Instruction order of one step (one wave per SIMD, so the wave's own
// order decides what overlaps): the four exchange reads and the first four
// key reads, then each score MFMA followed by the next key read; then eight
// transposing value reads, and each value MFMA followed by two more.  Keeping
// reads that far ahead of their MFMAs measured best against 2-8 key and
// 4-16 value reads ahead, and against one interleaving of both phases.
constexpr int kKeyAhead = 4, kValAhead = 8;
__device__ __forceinline__ void mw_schedule_scores() {
  __builtin_amdgcn_sched_group_barrier(0x100, 4 + kKeyAhead, 0);  // LDS reads
#pragma unroll
  for (int i = 0; i < 18; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    if (i + kKeyAhead < 18) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
}
__device__ __forceinline__ void mw_schedule_values() {
  __builtin_amdgcn_sched_group_barrier(0x100, kValAhead, 0);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (2 * i + kValAhead < 32) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  }
}

typedef __attribute__((address_space(3))) const char lds_cchar;
__device__ __forceinline__ u32x4 mw_read128(lds_cchar* p) {
  return *reinterpret_cast<__attribute__((address_space(3))) const u32x4*>(p);
}
__device__ __forceinline__ u32x2 mw_read_tr(lds_cchar* p) {
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  const v4i16 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16*)(p));
  return __builtin_bit_cast(u32x2, x);
}

template <class T, bool FLAT>
__global__ __launch_bounds__(64 * kMwWaves, 1) void mla_wide_kernel(MlaArgs a) {
  typedef typename T::vec8 vec8;
  __shared__ __attribute__((aligned(16))) uint16_t lds[kMwStages * kMwStageBytes / 2];
  // partial scores of one tile: sx[hb][dh][k][lane] = the lane's partial
  // scores 4k .. 4k + 3 of head block hb, dim half dh (16-byte accesses
  // consecutive across lanes)
  __shared__ __attribute__((aligned(16))) f32x4 sx[2][2][4][64];
  const int HG = a.H / 64;
  int hg, unit;
  if (!mla_unit(blockIdx.x, HG, FLAT ? a.pieces : a.units, hg, unit)) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int dh = w & 1, hb = w >> 1, h = lane >> 5, l32 = lane & 31;
  const int H = a.H;
  const int64_t rows = int64_t(a.B) * H;

  // Keys [lo, hi) of request b for this workgroup's 64 heads: split slot i
  // of the request's splits_b (final output when splits_b == 1).
  auto segment = [&](int b, int lo, int hi, int i, int splits_b) {
  const int64_t kb0 = a.kv_indptr[b];
  const int64_t row0 = int64_t(b) * H + 64 * hg;  // the workgroup's first head row
  const int n = hi - lo;
  const int ntiles = (n + kMwBK - 1) / kMwBK;
  // this lane's head row: head l32 of the wave's block
  const int64_t rowA = row0 + 32 * hb + l32;

  // Q^T operands of the eighteen contraction steps: head 32 hb + l32, dims
  // 288 dh + 16 u + 8 h .. +8.  Issued here and waited for together with the
  // first two tiles (run, below), so the two memory round trips overlap.
  u32x4 qa[18];
  {
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + rowA * kMlaD + 288 * dh + 8 * h;
#pragma unroll
    for (int u = 0; u < 18; ++u) qa[u] = ldg128(qp + 16 * u);
  }

  // direct-to-LDS loads: instruction x = w + 4k fills stage chunks
  // 64x .. 64x + 63; lane chunk q = 64x + lane is row q / 72, slot q % 72,
  // holding chunk slot ^ f(row) of the row
  int voff[kMwPerWave];
#pragma unroll
  for (int k = 0; k < kMwPerWave; ++k) {
    const int q = 64 * (w + kMwWaves * k) + lane;
    const int r = q / kMlaChunks, c = q % kMlaChunks;
    voff[k] = (r * kMlaChunks + (c ^ mw_swz(r))) * 16;
  }
  typedef int i32x4 __attribute__((ext_vector_type(4)));
  const uint64_t cbase = uint64_t(size_t(static_cast<const uint16_t*>(a.kv) + (kb0 + lo) * kMlaD));
  const uint32_t lds0 = uint32_t(size_t((__attribute__((address_space(3))) uint16_t*)lds)) + w * 1024;
  // A tile's loads are issued one at a time between the score MFMAs of the
  // step (dma_part), so that the wave never stalls on a full load queue; no
  // LDS access of the step touches the stage being filled (the barriers
  // that end each step order the rest), so the asm carries no memory
  // clobber and the compiler may keep LDS reads in flight across it.
  struct DmaTile {
    i32x4 rsv;
    uint32_t st;
  };
  auto dma_tile = [&](int tile) {
    const int key0 = tile * kMwBK;
    int left = n - key0;
    left = left < 0 ? 0 : (left > kMwBK ? kMwBK : left);
    const uint64_t addr = cbase + uint64_t(uint32_t(key0)) * (2 * kMlaD);
    DmaTile d;
    d.rsv = i32x4{__builtin_amdgcn_readfirstlane(int(uint32_t(addr))),
                  __builtin_amdgcn_readfirstlane(int(uint32_t(addr >> 32) & 0xffffu)),
                  __builtin_amdgcn_readfirstlane(left * 2 * kMlaD), 0x00020000};
    d.st = lds0 + uint32_t(tile % kMwStages) * kMwStageBytes;
    return d;
  };
  auto dma_part = [&](const DmaTile& d, int k) {
    __asm__ volatile(
        "s_mov_b32 m0, %0\n\t"
        "buffer_load_dwordx4 %1, %2, 0 offen lds"
        :
        : "s"(__builtin_amdgcn_readfirstlane(d.st + k * 1024 * kMwWaves)), "v"(voff[k]), "s"(d.rsv)
        : "m0");
  };
  auto dma = [&](int tile) {
    const DmaTile d = dma_tile(tile);
#pragma unroll
    for (int k = 0; k < kMwPerWave; ++k) dma_part(d, k);
  };

  // K operand reads (byte offsets in a stage): lane l32 reads key row l32,
  // chunk ch = 36 dh + 2 u + h, stored at slot ch ^ f(l32).  Chunks u and
  // u + 4 are 8 apart and f only touches the low three bits, so four
  // per-lane offsets and immediates cover the eighteen reads.
  int kofs[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) kofs[u] = 2 * (l32 * kMlaD + 8 * ((36 * dh + 2 * u + h) ^ mw_swz(l32)));
  // V^T operand (transposing reads): lane q + 4e of its 16-lane group
  // points at key row k0 + e (k0 = 16 t + 4 h, then + 8) and dims
  // 256 dh + 32 db + 16 g2 + 4 q; those rows have f = 2 e + h, and blocks
  // db and db + 2 are 8 chunks apart: two per-lane offsets (db even, odd)
  const int tq = lane & 3, te = (lane >> 2) & 3, g2 = (lane >> 4) & 1;
  int vofs[2];
#pragma unroll
  for (int d = 0; d < 2; ++d) {
    const int dim = 256 * dh + 32 * d + 16 * g2 + 4 * tq;
    vofs[d] = 2 * ((4 * h + te) * kMlaD + 8 * ((dim >> 3) ^ (2 * te + h)) + (dim & 7));
  }

  // O^T of the wave: head l32, dims 256 dh + 32 db + 8 (r / 4) + 4 h + r % 4
  f32x16 oa[8];
  float la = 0.f, mra = 0.f, mruna = -INFINITY;
  int flag = 0;
  const float c = fabsf(a.scale_log2);

  // LDS byte offsets are formed once per tile as (per-lane base + stage)
  // behind an empty asm, so that every read below is that base plus an
  // immediate (the compiler would otherwise keep one full address per read
  // and add the stage to each of them every tile).
  auto opaque = [](int v) {
    __asm__ volatile("" : "+v"(v));
    return v;
  };
  const int lds_base = int(uint32_t(size_t((__attribute__((address_space(3))) uint16_t*)lds)));

  // this wave's partial scores of the tile in stage `so` (its half of the
  // dims)
  // (with a tile to load: its nine loads go out after the odd MFMAs)
  auto scores = [&](int so, f32x16& sa, const DmaTile* d) {
#pragma unroll
    for (int r = 0; r < 16; ++r) sa[r] = 0.f;
    lds_cchar* kp[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) kp[u] = (lds_cchar*)(size_t)opaque(lds_base + so + kofs[u]);
#pragma unroll
    for (int u = 0; u < 18; ++u) {
      const u32x4 ka = mw_read128(kp[u & 3] + 128 * (u >> 2));
      sa = T::mfma32(as<vec8>(ka), as<vec8>(qa[u]), sa);
      if (d && (u & 1)) dma_part(*d, u >> 1);
    }
  };
  auto publish = [&](const f32x16& sa) {
#pragma unroll
    for (int k = 0; k < 4; ++k)
      sx[hb][dh][k][lane] = f32x4{sa[4 * k], sa[4 * k + 1], sa[4 * k + 2], sa[4 * k + 3]};
  };

  // One step of the pass (see the schedule above) for tile j; `last` marks
  // the chunk's last tile, whose keys past the chunk end are masked (kept
  // out of the loop so that the loop body is one basic block the compiler
  // can interleave).  Scores stay unscaled until the exponent: with the
  // scale c >= 0 (a negative scale was moved into the query signs), the
  // tile max is c times the max of the raw scores and each weight is
  // exp2(fma(s, c, -m)).
  f32x16 own;  // this wave's partial scores of the tile the step turns into weights
  int sv = 0, sk = kMwStageBytes;  // stages of tile j (values) and tile j + 1 (keys)
  auto step = [&](int j, bool exact, auto last) {
    // the partner's partial scores of tile j
    f32x4 o4[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) o4[k] = sx[hb][dh ^ 1][k][lane];
    const DmaTile dn = dma_tile(j + 3);
    // tile j + 1's partial scores (past the last tile: a stage of zeros or
    // stale rows, never used), with tile j + 3's loads
    f32x16 nxt;
    scores(sk, nxt, &dn);
    // tile j: the pair's partial scores added half 0 + half 1; keys of
    // sc[r]: j * 32 + 8 (r / 4) + 4 h + r % 4
    f32x16 sc;
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        sc[4 * k + e] = dh == 0 ? own[4 * k + e] + o4[k][e] : o4[k][e] + own[4 * k + e];
    bool valid[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      valid[r] = true;
      if constexpr (decltype(last)::value) valid[r] = j * kMwBK + 4 * h + 8 * (r >> 2) + (r & 3) < n;
    }
    float mx = valid[0] ? sc[0] : -INFINITY;
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, valid[r] ? sc[r] : -INFINITY);
    mx = max_halves(mx) * c;  // the tile's row max of head l32 (log2 units)
    if (!exact) {
      mruna = fmaxf(mruna, mx);
      // the reference: tile 0's row max (tile 0 holds a valid key)
      flag |= (j > 0) & (mx > mra + mw_overflow(T{}));
      mra = j == 0 ? mx : mra;
    }
    // weights: slots 8t .. 8t + 7 of the value update are sc[8t .. 8t + 7]
    vec8 pa[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      f32x8 p;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = fexp2(__builtin_fmaf(sc[8 * t + e], c, -mra));
        if constexpr (decltype(last)::value) p[e] = valid[8 * t + e] ? p[e] : 0.f;
      }
      la += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
      pa[t] = T::cvt8(p);
    }
    mw_schedule_scores();
    // every wave has read its partner's partials of tile j: the single
    // exchange buffer can take tile j + 1's
    __syncthreads();
    publish(nxt);
    // tile j's value update
    lds_cchar* vp[2] = {(lds_cchar*)(size_t)opaque(lds_base + sv + vofs[0]),
                        (lds_cchar*)(size_t)opaque(lds_base + sv + vofs[1])};
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        lds_cchar* p = vp[db & 1] + 128 * (db >> 1) + 2 * 16 * t * kMlaD;
        const u32x2 v0 = mw_read_tr(p);
        const u32x2 v1 = mw_read_tr(p + 2 * 8 * kMlaD);
        const u32x4 av = {v0[0], v0[1], v1[0], v1[1]};
        oa[db] = T::mfma32(as<vec8>(av), pa[t], oa[db]);
      }
    own = nxt;
    sv = sk;
    sk = sk == (kMwStages - 1) * kMwStageBytes ? 0 : sk + kMwStageBytes;
    mw_schedule_values();
    // vmcnt(9): tile j + 2 has arrived, tile j + 3's nine loads may still be
    // in flight
    static_assert(kMwPerWave == 9, "vmcnt immediate below");
    __builtin_amdgcn_s_waitcnt(0x0F79);
    __syncthreads();  // tile j + 1's partials and tile j + 2 published, stage j free
  };
  // One pass over the chunk (exact = 1: reference fixed from the start).
  auto run = [&](bool exact) {
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oa[db][r] = 0.f;
    la = 0.f;
    sv = 0;
    sk = kMwStageBytes;
    dma(0);
    dma(1);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): tiles 0 and 1 (and the queries) are in
    dma(2);
    if (!exact) {
      // a negative scale flips the sign of every query element instead (the
      // sign bit of both 16-bit formats is bit 15), so that c >= 0 below;
      // the empty asm keeps the flip after the wait above
      const uint32_t sgn = a.scale_log2 < 0.f ? 0x80008000u : 0u;
#pragma unroll
      for (int u = 0; u < 18; ++u) {
        __asm__ volatile("" : "+v"(qa[u]));
        qa[u] ^= sgn;
      }
    }
    __syncthreads();
    scores(0, own, nullptr);
    publish(own);
    __syncthreads();
    for (int j = 0; j < ntiles - 1; ++j) step(j, exact, std::false_type{});
    step(ntiles - 1, exact, std::true_type{});
    // the last steps' loads (past the chunk: zeros) land before the stages
    // are reused
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  };
  // any wave's flag, through the (now free) exchange buffer
  auto any_flag = [&](int f) {
    int* fl = reinterpret_cast<int*>(&sx[0][0][0][0]);
    const uint64_t bal = __ballot(f != 0);
    if (lane == 0) fl[w] = bal != 0;
    __syncthreads();
    const int r = fl[0] | fl[1] | fl[2] | fl[3];
    __syncthreads();  // every wave has read the flags before the buffer is reused
    return r;
  };
  run(false);
  if (any_flag(flag)) {  // a score far above the first tile's max
    mra = mruna;
    run(true);
  }

  // The wave's output block (32 heads x 256 dims) goes out through LDS (the
  // stages are free once every wave has passed the last step's barrier):
  // the accumulator layout gives each lane 4 dims of a head per register
  // group, which would make every store instruction touch 32 rows; read
  // back from a 32 x 528-byte area per wave, each half-wave holds 512
  // contiguous bytes of one head row.  Final rows are written in the
  // inputs' 16-bit type, split partials in fp16 with each 128-dim quarter
  // scaled by its power of two (mla_part_exp).
  auto store = [&](const f32x16 (&o)[8], float l, float mref, int64_t row) {
    l = sum_halves(l);
    const float inv = 1.f / l;
    typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
    typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
    __attribute__((address_space(3))) char* blk =
        (__attribute__((address_space(3))) char*)lds + w * (32 * kMwOutRow);
    const int64_t hrow0 = row0 + 32 * hb + h;  // store k below: head 2k + h of the block
    const bool final_rows = splits_b == 1;
    // quarters 2 dh + qq of the row: value blocks db = 4 qq .. 4 qq + 3,
    // held by this lane and its partner l ^ 32
    int e[2] = {0, 0};
    if (!final_rows) {
#pragma unroll
      for (int qq = 0; qq < 2; ++qq) {
        float amax = 0.f;
#pragma unroll
        for (int db = 4 * qq; db < 4 * qq + 4; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) amax = fmaxf(amax, fabsf(o[db][r]));
        e[qq] = mla_part_exp(max_halves(amax) * inv);
      }
    }
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        f32x8 y;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          y[k] = final_rows ? o[db][4 * g4 + k] * inv
                            : __builtin_amdgcn_ldexpf(o[db][4 * g4 + k] * inv, -e[db >> 2]);
          y[4 + k] = 0.f;
        }
        const u32x4 bits = final_rows ? __builtin_bit_cast(u32x4, T::cvt8(y))
                                      : __builtin_bit_cast(u32x4, F16::cvt8(y));
        *reinterpret_cast<lds_u32x2*>(blk + l32 * kMwOutRow + 2 * (32 * db + 8 * g4 + 4 * h)) =
            u32x2{bits[0], bits[1]};
      }
    // LDS accesses of one wave complete in issue order; the fences keep the
    // compiler from moving the reads above the writes
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    uint16_t* base = final_rows ? static_cast<uint16_t*>(a.o) : a.o_part + int64_t(i) * rows * kMlaDc;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const u32x4 v = *reinterpret_cast<lds_u32x4*>(blk + (2 * k + h) * kMwOutRow + 16 * l32);
      *reinterpret_cast<u32x4*>(base + (hrow0 + 2 * k) * kMlaDc + 256 * dh + 8 * l32) = v;
    }
    if (final_rows) {
      if (a.lse && dh == 0 && h == 0) a.lse[row] = (mref + flog2(l)) * kLn2;
    } else {
      if (h == 0)
        *reinterpret_cast<f32x2*>(a.x_part + (int64_t(i) * rows + row) * 4 + 2 * dh) =
            f32x2{__builtin_amdgcn_ldexpf(1.f, e[0]), __builtin_amdgcn_ldexpf(1.f, e[1])};
      if (dh == 0 && h == 0) {
        a.m_part[int64_t(i) * rows + row] = mref * kLn2;
        a.l_part[int64_t(i) * rows + row] = l;
      }
    }
  };
  store(oa, la, mra, rowA);
  __syncthreads();  // (flat plan) the next segment's first loads reuse the stages
  };

  if constexpr (!FLAT) {
    // chunk plan: split i of request b covers its keys [i c, (i + 1) c);
    // unit b s + i for equal lengths, packed units (mla_packed_unit) for
    // ragged ones
    const int64_t c = a.chunk;
    int b = unit / a.s, i = unit % a.s;
    if (a.packed && !mla_packed_unit(a, unit, lane, b, i)) return;  // past the last unit
    const int64_t kb0 = a.kv_indptr[b], kb1 = a.kv_indptr[b + 1];
    const int n_b = int(kb1 - kb0);
    if (n_b <= 0) {  // empty request: O = 0, LSE = -inf
      if (i != 0) return;  // (direct mapping: written by its split 0)
      const int64_t row0 = int64_t(b) * H + 64 * hg;
      typename T::elem* o = static_cast<typename T::elem*>(a.o) + row0 * kMlaDc;
      for (int e = tid; e < 64 * kMlaDc; e += 64 * kMwWaves) o[e] = typename T::elem(0.f);
      if (a.lse && tid < 64) a.lse[row0 + tid] = -INFINITY;
      return;
    }
    const int lo = int(int64_t(i) * c);
    if (lo >= n_b) return;  // a split the request does not have (direct mapping)
    const int hi = lo + c < n_b ? int(lo + c) : n_b;
    segment(b, lo, hi, i, int(min((int64_t(n_b) + c - 1) / c, int64_t(a.s))));
  } else {
    // flat plan: piece p = packed cache rows [p c, (p + 1) c); split i of a
    // request is its intersection with the i-th piece it overlaps.  The
    // pieces' request segments are reduced one after the other; requests
    // inside one piece are final here, the others leave partials for the
    // merge (which also writes empty requests).
    const int64_t c = a.chunk, p = unit;
    const int64_t pos0 = p * c, pos1 = pos0 + c < a.total_kv ? pos0 + c : a.total_kv;
    if (pos0 >= pos1) return;
    // first request that may hold row pos0: (indptr entries <= pos0) - 1,
    // counted 64 entries per step across the lanes
    int cnt = 0;
    for (int j0 = 0; j0 <= a.B; j0 += 64) {
      const int j = j0 + lane;
      cnt += __popcll(__ballot(j <= a.B && int64_t(a.kv_indptr[j <= a.B ? j : a.B]) <= pos0));
    }
    for (int b = __builtin_amdgcn_readfirstlane(cnt > 0 ? cnt - 1 : 0); b < a.B; ++b) {
      const int64_t r0 = a.kv_indptr[b], r1 = a.kv_indptr[b + 1];
      if (r0 >= pos1) break;
      const int64_t lo = r0 > pos0 ? r0 : pos0, hi = r1 < pos1 ? r1 : pos1;
      if (lo >= hi) continue;  // empty request, or one that ends before pos0
      const int splits_b = int((r1 - 1) / c - r0 / c) + 1;
      const int i = int(p - r0 / c);
      // (with a consistent indptr 0 <= i < s always holds; otherwise nothing
      // is written outside the workspace)
      if (splits_b > 1 && (i < 0 || i >= a.s)) continue;
      segment(b, int(lo - r0), int(hi - r0), i, splits_b);
    }
  }
}

// ---------------------------------------------------------------------------
// Merge of the split partials (512-wide latent outputs), the log-sum-exp
// merge of the Split operator: M = max m_i, w_i = l_i e^{m_i - M},
// O = sum w_i o_i / sum w_i, LSE = M + ln sum w_i.  One wave per (request,
// head) row; lane l holds dims 8l .. 8l + 7 (quarter l / 16 of the row), so
// one split's partial row is a single 1 KB read by the wave (one 16-byte
// load per lane), and the splits arrive in batches of SB whose loads are
// all issued before the first is used (one memory round trip per batch; a
// batch's slots past the last split re-read the last one and weigh it 0).
// The partial rows are fp16 with a power-of-two scale per quarter
// (mla_part_exp); lane j of the wave forms split j's weight times each of
// its four scales, and every lane takes the one of its own quarter.  A
// request's split count comes from kv_indptr and the chunk (or piece)
// length, capped at s, so no read leaves the workspace; requests held by
// one split were written by the kernel itself.  An empty request of the
// flat plan is written here (O = 0, LSE = -inf); the chunk plan's kernel
// writes its own.
// ---------------------------------------------------------------------------
template <class T, int SB>
__global__ __launch_bounds__(256) void mla_merge_kernel(MlaArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t rows = int64_t(a.B) * a.H;
  // (the wave index read as uniform: the row's indptr entries and split
  // count then live in scalar registers and the loops stay uniform)
  const int64_t row = int64_t(blockIdx.x) * 4 + __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  if (row >= rows) return;
  const int b = int(row / a.H);
  const int64_t kb0 = a.kv_indptr[b], kb1 = a.kv_indptr[b + 1];
  const int64_t c = a.chunk;
  int64_t n64 = 0;
  if (c > 0 && kb1 > kb0) n64 = a.flat ? (kb1 - 1) / c - kb0 / c + 1 : (kb1 - kb0 + c - 1) / c;
  const int n = int(n64 < a.s ? n64 : a.s);
  typename T::elem* orow = static_cast<typename T::elem*>(a.o) + row * kMlaDc + 8 * lane;
  if (n == 0 && a.flat) {
    *reinterpret_cast<u32x4*>(orow) = u32x4{0u, 0u, 0u, 0u};
    if (a.lse && lane == 0) a.lse[row] = -INFINITY;
  }
  if (n <= 1) return;
  const int qt = lane >> 4;  // the lane's quarter of the row

  // splits [i0, i0 + cnt) of one batch of 64: partial rows read SB at a
  // time, each weighed by lane j's weight for this lane's quarter
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  u32x4 xr[SB];
  auto load = [&](int i0, int j0, int cnt) {
    const uint16_t* op = a.o_part + (int64_t(i0) * rows + row) * kMlaDc + 8 * lane;
#pragma unroll
    for (int j = 0; j < SB; ++j) {
      const int jj = j0 + j < cnt ? j0 + j : cnt - 1;
      xr[j] = *reinterpret_cast<const u32x4*>(op + int64_t(jj) * rows * kMlaDc);
    }
  };
  // Lane j of a batch of 64 splits publishes split j's weight times its
  // four quarter scales in an LDS table (zero past the batch's count, and
  // in the padding past 64 that a last read of SB splits may reach); each
  // lane then reads its quarter's weights four splits at a time.
  constexpr int WT = 64 + 32;  // table row: 64 splits, then zeros
  static_assert(SB <= 32, "a batch's reads stay inside a table row");
  __shared__ __attribute__((aligned(16))) float wtab[4][4][WT];  // [wave][quarter][split]
  float* wt = &wtab[__builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6))][0][0];
  if (lane < 32) {
#pragma unroll
    for (int k = 0; k < 4; ++k) wt[WT * k + 64 + lane] = 0.f;
  }
  auto wave_sync = [] {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  auto publish = [&](f32x4 wq) {
    wave_sync();  // the previous batch's reads are done
#pragma unroll
    for (int k = 0; k < 4; ++k) wt[WT * k + lane] = wq[k];
    wave_sync();
  };
  auto add = [&](int j0) {
    static_assert(SB % 4 == 0, "weights are read four at a time");
#pragma unroll
    for (int j4 = 0; j4 < SB; j4 += 4) {
      const f32x4 w4 = *reinterpret_cast<const f32x4*>(wt + WT * qt + j0 + j4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const f32x8 x = __builtin_convertvector(as<f16x8>(xr[j4 + e]), f32x8);
        acc0 += w4[e] * f32x4{x[0], x[1], x[2], x[3]};
        acc1 += w4[e] * f32x4{x[4], x[5], x[6], x[7]};
      }
    }
  };
  // the first 64 splits' (m, l, scales) and the first SB partial rows go
  // out together, before any of them is used
  const int cnt0 = n < 64 ? n : 64;
  float m0 = -INFINITY, l0 = 0.f;
  f32x4 x0 = {0.f, 0.f, 0.f, 0.f};
  if (lane < cnt0) {
    const int64_t k = int64_t(lane) * rows + row;
    m0 = a.m_part[k];
    l0 = a.l_part[k];
    x0 = *reinterpret_cast<const f32x4*>(a.x_part + 4 * k);
  }
  load(0, 0, cnt0);
  float M = m0;
  for (int i = 64 + lane; i < n; i += 64) M = fmaxf(M, a.m_part[int64_t(i) * rows + row]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, shfl_xor(M, off));
  float wsum = 0.f;
  {
    const float wi = lane < cnt0 ? l0 * fexp2((m0 - M) * kLog2e) : 0.f;
    wsum += wi;
    publish(wi * x0);
    add(0);
    for (int j0 = SB; j0 < cnt0; j0 += SB) {
      load(0, j0, cnt0);
      add(j0);
    }
  }
  for (int i0 = 64; i0 < n; i0 += 64) {  // more than 64 splits
    const int cnt = n - i0 < 64 ? n - i0 : 64;
    float wi = 0.f;
    f32x4 xi = {0.f, 0.f, 0.f, 0.f};
    if (lane < cnt) {
      const int64_t k = int64_t(i0 + lane) * rows + row;
      wi = a.l_part[k] * fexp2((a.m_part[k] - M) * kLog2e);
      xi = *reinterpret_cast<const f32x4*>(a.x_part + 4 * k);
    }
    wsum += wi;
    publish(wi * xi);
    for (int j0 = 0; j0 < cnt; j0 += SB) {
      load(i0, j0, cnt);
      add(j0);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) wsum += shfl_xor(wsum, off);
  const float inv = 1.f / wsum;
  const f32x8 y = {acc0[0] * inv, acc0[1] * inv, acc0[2] * inv, acc0[3] * inv,
                   acc1[0] * inv, acc1[1] * inv, acc1[2] * inv, acc1[3] * inv};
  *reinterpret_cast<u32x4*>(orow) = __builtin_bit_cast(u32x4, T::cvt8(y));
  if (a.lse && lane == 0) a.lse[row] = M + flog2(wsum) * kLn2;
}

template <class T>
static hipError_t launch_mla_t(const MlaArgs& a, hipStream_t st) {
  if (a.flat) {  // the flat plan (many-head kernel only)
    const int64_t nwg = 8 * (a.H / 64) * ((int64_t(a.pieces) + 7) / 8);
    if (a.pieces > 0 && a.total_kv > 0)
      hipLaunchKernelGGL((mla_wide_kernel<T, true>), dim3(unsigned(nwg)), dim3(64 * kMwWaves), 0, st, a);
  } else if (mla_wide(a.H)) {
    const int64_t nwg = 8 * (a.H / 64) * ((int64_t(a.units) + 7) / 8);
    hipLaunchKernelGGL((mla_wide_kernel<T, false>), dim3(unsigned(nwg)), dim3(64 * kMwWaves), 0, st, a);
  } else {
    const int HG = (a.H + 15) / 16;
    const int64_t nwg = 8 * HG * ((int64_t(a.s) * a.B + 7) / 8);
    hipLaunchKernelGGL((mla_decode_kernel<T>), dim3(unsigned(nwg)), dim3(kMlaThreads), 0, st, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || (a.s == 1 && !a.flat)) return e;
  const int64_t rows = int64_t(a.B) * a.H;
  const dim3 grid(unsigned((rows + 3) / 4));
  if (a.s <= 8) hipLaunchKernelGGL((mla_merge_kernel<T, 8>), grid, dim3(256), 0, st, a);
  else if (a.s <= 16) hipLaunchKernelGGL((mla_merge_kernel<T, 16>), grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL((mla_merge_kernel<T, 20>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_mla_decode(const MlaArgs& a, hipStream_t st) {
  return a.dtype == 1 ? launch_mla_t<BF16>(a, st) : launch_mla_t<F16>(a, st);
}

}  // namespace rattn
