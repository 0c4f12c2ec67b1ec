// bsr_rows.hip -- row-wise block-sparse prefill on gfx950.
//
// The row kernel of the STOF explainer ("Accelerating Sparse Transformer
// Inference on GPU", 技術概要, "デュアルカーネル戦略"): queries sliced by
// rows, cross-lane operations inside one wave, no synchronisation between
// waves.  It reads the same two-level mask as the block-wise kernel (BSR
// outer tiles plus one uint64 per 8x8 inner tile, "2 段階ストレージ形式").
//
// Each wave owns 16 query rows -- two inner-tile rows of an outer-tile row --
// of one head, and walks on its own the 16-key column blocks of its row's
// stored outer tiles in which its rows hold at least one valid element: all
// four blocks of a full tile, and of a part tile those whose two bitmap rows
// are not zero.  A block costs two 16x16 MFMA passes over its keys:
//   S^T = K Q^T on 16x16x32 MFMAs, K rows loaded straight into registers;
//   masking from the bitmap nibble each lane needs (4 keys of its row);
//   online softmax per query row, the row max combined over the four 16-lane
//   rows that hold the row's 16 keys, the sum kept per lane until the end;
//   O^T += V^T P^T on 16x16x16 MFMAs, P^T taken from the S^T accumulator as
//   it stands and V^T read transposed from a 16-row block the wave stages in
//   its own LDS slot.
// The next block's K, V and bitmap word are loaded while the current one is
// computed.  With 16-key granularity the kernel skips what the block-wise
// kernel, working on whole 64x64 tiles, has to compute.
#include "attn_core.hpp"
#include "launch.hpp"

namespace rattn {

// x combined with lanes l ^ 16, l ^ 32 and l ^ 48, in every lane.  The
// 16-lane swap exchanges the odd rows of one copy with the even rows of the
// other, leaving each lane its own value and its l ^ 16 partner's; the
// 32-lane swap (max_halves / sum_halves) then pairs the halves.
__device__ __forceinline__ float max_rows4(float x) {
  const int b = __float_as_int(x);
  const auto r = __builtin_amdgcn_permlane16_swap(b, b, false, false);
  return max_halves(fmaxf(__int_as_float(r[0]), __int_as_float(r[1])));
}
__device__ __forceinline__ float sum_rows4(float x) {
  const int b = __float_as_int(x);
  const auto r = __builtin_amdgcn_permlane16_swap(b, b, false, false);
  return sum_halves(__int_as_float(r[0]) + __int_as_float(r[1]));
}

// v_mfma_f32_16x16x16 (four 16-bit operands per lane: k-slots
// 4 (l / 16) + 0..3) and the fp32 -> 16-bit conversion of four values.
template <class T>
__device__ __forceinline__ f32x4 mfma16k16(u32x2 a, u32x2 b, f32x4 c);
template <>
__device__ __forceinline__ f32x4 mfma16k16<BF16>(u32x2 a, u32x2 b, f32x4 c) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(v4s, a),
                                                   __builtin_bit_cast(v4s, b), c, 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x4 mfma16k16<F16>(u32x2 a, u32x2 b, f32x4 c) {
  typedef _Float16 v4h __attribute__((ext_vector_type(4)));
  return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(v4h, a),
                                               __builtin_bit_cast(v4h, b), c, 0, 0, 0);
}
template <class T>
__device__ __forceinline__ u32x2 cvt4(f32x4 x) {
  typedef typename T::elem e4 __attribute__((ext_vector_type(4)));
  return __builtin_bit_cast(u32x2, __builtin_convertvector(x, e4));
}

template <class T, int D>
__global__ __launch_bounds__(256) void bsr_rows_kernel(BsrArgs a) {
  typedef typename T::vec8 vec8;
  typedef Swz<D> S;
  constexpr int NU = D / 32;     // 32-dim slices of the score contraction
  constexpr int NDB = D / 16;    // 16-dim blocks of O^T
  constexpr int CPR = D / 8;     // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;  // rows per 64-lane load
  constexpr int NV = 16 / RPI;   // V loads per lane per 16-key block
  __shared__ __attribute__((aligned(16))) uint16_t vbuf[4][16 * D];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i = lane & 15, gq = lane >> 4;
  int qblk, hq;
  bsr_block_head(a.num_blocks, a.Hq, qblk, hq);
  const int b = blockIdx.z;
  const int64_t L = a.L;
  const int hk = hq / a.G;
  const int mrow = (hq / a.heads_per_mask) * (a.num_blocks + 1) + qblk;  // this head's mask
  const int f0 = a.full_indptr[mrow], n_full = a.full_indptr[mrow + 1] - f0;
  const int p0 = a.part_indptr[mrow], n_part = a.part_indptr[mrow + 1] - p0;
  const int n_ot = n_full + n_part;
  const int q = qblk * 64 + 16 * w + i;  // the lane's query row: a column of S^T
  const int row_stride = a.Hkv * D;
  const uint16_t* kbase = static_cast<const uint16_t*>(a.k) + int64_t(b) * L * row_stride + int64_t(hk) * D;
  const uint16_t* vbase = static_cast<const uint16_t*>(a.v) + int64_t(b) * L * row_stride + int64_t(hk) * D;
  const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + ((int64_t(b) * L + q) * a.Hq + hq) * D;
  uint16_t* const vw = vbuf[w];
  const float c = a.scale_log2;

  // Q^T operand: lane l holds dims 32u + 8 (l / 16) .. +8 of query l % 16
  u32x4 qv[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) qv[u] = ldg128(qrow + 32 * u + 8 * gq);

  f32x4 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;

  // Cursor over the wave's blocks (uniform): outer tile t of the row's full
  // then part list, and the blocks of it still to visit.
  int t = -1, rem = 0, kblk = 0, pid = -1;
  auto next = [&](int& u_kblk, int& u_kb, int& u_pid) -> bool {
    while (rem == 0) {
      if (++t >= n_ot) return false;
      if (t < n_full) {
        kblk = a.full_kblock[f0 + t];
        pid = -1;
        rem = 0xF;
      } else {
        pid = p0 + t - n_full;
        kblk = a.part_kblock[pid];
        // bitmap words of inner-tile rows 2w and 2w + 1: 16w + ic, 16w + 8 + ic
        const uint64_t* wp = a.part_bits + int64_t(pid) * 64 + 16 * w;
        rem = 0;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
          if (wp[2 * kb] | wp[2 * kb + 1] | wp[8 + 2 * kb] | wp[9 + 2 * kb]) rem |= 1 << kb;
      }
    }
    u_kb = __builtin_ctz(rem);
    rem &= rem - 1;
    u_kblk = kblk;
    u_pid = pid;
    return true;
  };

  struct Regs {
    u32x4 k[NU];
    u32x4 v[NV];
    uint64_t word;
  };
  auto issue = [&](Regs& R, int u_kblk, int u_kb, int u_pid) {
    const int key0 = u_kblk * 64 + u_kb * 16;
    // K: lane l takes key key0 + l % 16, dims 32u + 8 (l / 16) .. +8
    const uint16_t* kp = kbase + int64_t(key0 + i) * row_stride + 8 * gq;
#pragma unroll
    for (int u = 0; u < NU; ++u) R.k[u] = ldg128(kp + 32 * u);
    // V: rows RPI x + l / CPR, chunk l % CPR
#pragma unroll
    for (int x = 0; x < NV; ++x)
      R.v[x] = ldg128(vbase + int64_t(key0 + RPI * x + lane / CPR) * row_stride + 8 * (lane % CPR));
    // bitmap word of the lane's inner tile: row 2w + i / 8, column 2 kb + gq / 2
    R.word = u_pid >= 0 ? a.part_bits[int64_t(u_pid) * 64 + (2 * w + i / 8) * 8 + 2 * u_kb + gq / 2]
                        : ~0ull;
  };
  auto compute = [&](const Regs& R) {
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < NU; ++u) s = T::mfma16(as<vec8>(R.k[u]), as<vec8>(qv[u]), s);
    // s[r]: query i, key 4 gq + r of the block; its bit is r8 * 8 + c8 with
    // r8 = i % 8 and c8 = 4 (gq % 2) + r in the word loaded above
    // (bit r of the nibble, sign-extended, selects the score or -inf)
    const int nib = int(uint32_t(R.word >> ((i & 7) * 8 + 4 * (gq & 1))));
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t keep = uint32_t(__builtin_amdgcn_sbfe(nib, r, 1));
      s[r] = __uint_as_float((__float_as_uint(s[r]) & keep) | (0xFF800000u & ~keep));
    }
    const float mx = max_rows4(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]))) * c;
    // lazy rescale (see kRescaleSlack); uniform over the lanes of a query
    const bool need = mx > m + kRescaleSlack;
    if (__any(need)) {
      const float m_new = need ? mx : m;
      const float alpha = need ? fexp2(m - m_new) : 1.f;
#pragma unroll
      for (int db = 0; db < NDB; ++db) o[db] *= alpha;
      l *= alpha;
      m = m_new;
    }
    const float mref = m == -INFINITY ? 0.f : m;
    f32x4 p;
#pragma unroll
    for (int r = 0; r < 4; ++r) p[r] = fexp2(__builtin_fmaf(s[r], c, -mref));
    l += (p[0] + p[1]) + (p[2] + p[3]);
    const u32x2 pb = cvt4<T>(p);
    // stage V in the wave's slot, 16-byte chunks swizzled per row
#pragma unroll
    for (int x = 0; x < NV; ++x) {
      const int row = RPI * x + lane / CPR, chunk = lane % CPR;
      *reinterpret_cast<u32x4*>(vw + row * D + 8 * (chunk ^ S::fv(row))) = R.v[x];
    }
    // O^T += V^T P^T: lane i of row group gq supplies row 4 gq + i / 4, dims
    // 16 db + 4 (i % 4) .. +4, and receives keys 4 gq .. +4 of dim 16 db + i
    const int vrow = 4 * gq + i / 4;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int dim = 16 * db + 4 * (i & 3);
      const int off = 2 * (vrow * D + 8 * ((dim >> 3) ^ S::fv(vrow)) + (dim & 7));
      o[db] = mfma16k16<T>(lds_tr4(vw, off), pb, o[db]);
    }
  };

  Regs R0, R1;
  int kk0, kb0, pd0, kk1, kb1, pd1;
  bool v0 = next(kk0, kb0, pd0);
  if (v0) issue(R0, kk0, kb0, pd0);
  while (v0) {
    const bool v1 = next(kk1, kb1, pd1);
    if (v1) issue(R1, kk1, kb1, pd1);
    compute(R0);
    if (!v1) break;
    v0 = next(kk0, kb0, pd0);
    if (v0) issue(R0, kk0, kb0, pd0);
    compute(R1);
  }

  // epilogue: the row's sum over its four row groups; O^T lane l holds
  // dims 16 db + 4 (l / 16) + r of query l % 16
  const float lt = sum_rows4(l);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  uint16_t* orow = static_cast<uint16_t*>(a.o) + ((int64_t(b) * L + q) * a.Hq + hq) * D;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
    *reinterpret_cast<u32x2*>(orow + 16 * db + 4 * gq) = cvt4<T>(o[db] * inv);
  if (a.lse && gq == 0)
    a.lse[(int64_t(b) * L + q) * a.Hq + hq] = lt > 0.f ? (m + flog2(lt)) * kLn2 : -INFINITY;
}

hipError_t launch_prefill_bsr_rows(const BsrArgs& a, hipStream_t st) {
  const dim3 grid(a.num_blocks, a.Hq, a.B);
  if (a.dtype == 1) {  // bf16, else f16
    if (a.D == 64) hipLaunchKernelGGL((bsr_rows_kernel<BF16, 64>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((bsr_rows_kernel<BF16, 128>), grid, dim3(256), 0, st, a);
  } else {
    if (a.D == 64) hipLaunchKernelGGL((bsr_rows_kernel<F16, 64>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((bsr_rows_kernel<F16, 128>), grid, dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace rattn
