// Gate and top-k ("MoBA: Mixture of Block Attention for Long-Context LLMs", paper
// summary page, section "Approach": score each block by the inner product of the
// query with the block's mean-pooled key, route each query to its top-k blocks plus
// its own current block, causally; README bullet "Parameter-less Gating Mechanism").
// Like FlashTopK in the FlashMoBA story (hyper.ai), the T x nb score matrix is never
// written: scores live only in MFMA accumulators.
//
// Readings: topk counts the current block, so topk-1 history blocks compete; only
// blocks j < c = t / block compete; ties go to the lower block index; rows with
// c <= topk-1 take every block 0..c without scoring (their queries are never read).
//
// Mapping.  A wavefront owns 64 consecutive tokens of one query head h (kv-head g)
// and computes S^T = C Q^T on MFMA 32x32x16 for two tiles of 32 queries (rows = 32
// blocks, columns = 32 queries).  The centroid is float32; it enters the MFMA as bf16
// hi + bf16 lo (two products into one float32 accumulator), the query is bf16 already.
// In each tile lane l holds 16 scores of query l%32 (blocks (i/4)*8 + (l/32)*4 + i%4);
// one lane-half swap per accumulator register then gives lane l all 32 scores of
// query t0 + l, so every lane ranks one row on its own and the wavefront's idx rows
// are one contiguous run.
//
// Ranking.  Each score becomes a 32-bit key whose high bits order like the float and
// whose low nbits hold (mask - j), so larger key = better, and exactly equal scores
// rank the lower block first.  Scores closer than ~2^-(23-nbits) relative compare
// as equal (well inside the 1e-3-relative near-tie band).  Per 32-block tile a lane
// sorts its keys in two halves of 16 (odd-even merge networks), merges them, and
// merges the result into a running sorted top-KHMAX list (KHMAX = 16, 32 or 64;
// bitonic merges).  No branch depends on the data, so the wavefront never diverges.
#include "moba_internal.h"

namespace moba {

namespace {

// jbits = mask - j: the block's rank bits
__device__ __forceinline__ uint32_t gate_key(float s, uint32_t jbits, uint32_t mask) {
  const uint32_t u = __float_as_uint(s + 0.f);  // -0 + 0 = +0: ranks like +0
  // negative: all bits flipped; non-negative: sign bit set -> unsigned order = float order
  const uint32_t m = (uint32_t)((int32_t)u >> 31) | 0x80000000u;
  return ((u ^ m) & ~mask) | jbits;
}

template <int N>
__device__ __forceinline__ void cas_desc(uint32_t (&a)[N], int i, int k) {
  const uint32_t x = a[i], y = a[k];
  a[i] = max(x, y);
  a[k] = min(x, y);
}

// Batcher's odd-even merge sort network for 16 keys (63 comparators, against the
// bitonic network's 80), built at compile time.  Comparator (a, b), a < b, leaves the
// larger key at a, so the network sorts descending.
struct SortNet16 {
  int n;
  unsigned char a[63], b[63];
};
constexpr void oem_merge(SortNet16& net, int lo, int hi, int r) {
  const int step = r * 2;
  if (step < hi - lo) {
    oem_merge(net, lo, hi, step);
    oem_merge(net, lo + r, hi, step);
    for (int i = lo + r; i < hi - r; i += step) {
      net.a[net.n] = (unsigned char)i;
      net.b[net.n] = (unsigned char)(i + r);
      ++net.n;
    }
  } else {
    net.a[net.n] = (unsigned char)lo;
    net.b[net.n] = (unsigned char)(lo + r);
    ++net.n;
  }
}
constexpr void oem_sort(SortNet16& net, int lo, int hi) {
  if (hi - lo >= 1) {
    const int mid = lo + (hi - lo) / 2;
    oem_sort(net, lo, mid);
    oem_sort(net, mid + 1, hi);
    oem_merge(net, lo, hi, 1);
  }
}
constexpr SortNet16 make_sort16() {
  SortNet16 net{};
  oem_sort(net, 0, 15);
  return net;
}
constexpr SortNet16 kSort16 = make_sort16();
static_assert(kSort16.n == 63, "odd-even merge sort of 16 keys has 63 comparators");

__device__ __forceinline__ void sort16_desc(uint32_t (&a)[16]) {
#pragma unroll
  for (int i = 0; i < kSort16.n; ++i) cas_desc(a, kSort16.a[i], kSort16.b[i]);
}

// a bitonic sequence -> sorted descending
template <int N>
__device__ __forceinline__ void bitonic_merge_desc(uint32_t (&a)[N]) {
#pragma unroll
  for (int jj = N >> 1; jj > 0; jj >>= 1) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int ixj = i ^ jj;
      if (ixj > i) cas_desc(a, i, ixj);
    }
  }
}

// full bitonic sort, ascending, of signed ints
template <int N>
__device__ __forceinline__ void bitonic_sort_asc(int (&a)[N]) {
#pragma unroll
  for (int kk = 2; kk <= N; kk <<= 1) {
#pragma unroll
    for (int jj = kk >> 1; jj > 0; jj >>= 1) {
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const int ixj = i ^ jj;
        if (ixj > i) {
          const int x = a[i], y = a[ixj];
          const bool up = (i & kk) == 0;
          a[i] = up ? min(x, y) : max(x, y);
          a[ixj] = up ? max(x, y) : min(x, y);
        }
      }
    }
  }
}

}  // namespace

// Query operands of one chunk (64 tokens t0 .. t0+63 of head h of a sequence of T
// tokens starting at packed token tok0): tile qt, k-step s holds dims 16*s + 8*hf ..
// +7 of token t0 + 32*qt + n.  Loads go through a buffer descriptor of the chunk's rows
// (zero size when not needed), so rows past T read as zeros.
template <int D>
__device__ __forceinline__ void gate_load_q(bf16x8_t (&bq)[2][D / 16],
                                            const uint16_t* __restrict__ q, int T, int hq,
                                            int tok0, int h, int t0, bool needed) {
  const int lane = threadIdx.x & 63, n = lane & 31, hf = lane >> 5;
  const uint16_t* base = q + ((size_t)((size_t)tok0 + t0) * hq + h) * D;
  const int rows = min(64, T - t0);
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(base), (short)0,
      needed ? (int)(rows * hq * D * sizeof(uint16_t)) : 0, 0x00020000);
#pragma unroll
  for (int qt = 0; qt < 2; ++qt)
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      const int off = ((32 * qt + n) * hq * D + 16 * s + 8 * hf) * (int)sizeof(uint16_t);
      bq[qt][s] = as_bf16x8(__builtin_bit_cast(
          u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, 0, 0)));
    }
}

struct GateChunk {
  int b, h, t0;
  int T, tok0;   // the sequence's length and first packed token
  size_t lrow;   // idx row of (b, h, t = 0), in rows of topk
  bool compete;  // some row has more causal history blocks than slots
};

// chunk (b, h, t0) of a sequence; T is the longest sequence (the chunk grid)
__device__ __forceinline__ GateChunk gate_chunk_make(const SeqMap& sq, int b, int h, int t0,
                                                     int hq, int block, int KH) {
  GateChunk k;
  k.b = b;
  k.h = h;
  k.t0 = t0;
  k.T = sq.len(b);
  k.tok0 = sq.tok0(b);
  k.lrow = sq.lrow(b, h, hq);
  k.compete = KH > 0 && min(k.t0 + 63, k.T - 1) / block > KH;
  return k;
}

// rows of a chunk that need no score: with history slots, rows whose every causal
// block is selected (0..c, then -1); with none (topk == 1), just the current block
__device__ __forceinline__ void gate_all_blocks(const GateChunk& k, int block, int topk,
                                                int32_t* __restrict__ idx) {
  const int t = k.t0 + (threadIdx.x & 63);
  if (t < k.T) {
    const int c = t / block;
    int32_t* row = idx + (k.lrow + t) * topk;
    if (topk == 1) {
      row[0] = c;
      return;
    }
    for (int p = 0; p < topk; ++p) row[p] = p <= c ? p : -1;
  }
}

// LDS image of one kv-head's centroids: the bf16 hi rows then the lo rows, each row
// padded to CS bytes so that the 32 rows an MFMA operand read touches spread over the
// banks.
template <int D>
struct CentLds {
  static constexpr int CS = 2 * D + 16;
  static constexpr int MAX_NB = 96;
  static constexpr int BYTES = 2 * MAX_NB * CS;
};

// Rank one chunk (its rows compete) with its query operands bq.  The centroids come
// from global memory, or from the workgroup's LDS image lds (nb <= CentLds::MAX_NB).
template <int D, int KHMAX, bool CLDS, bool ONE = false>
__device__ __forceinline__ void gate_chunk(const bf16x8_t (&bq)[2][D / 16], const GateChunk& k,
                                           const uint16_t* __restrict__ chi,
                                           const uint16_t* __restrict__ clo,
                                           const char* __restrict__ lds, int hq,
                                           int hkv, int block, int nb, int topk, int nbits,
                                           int32_t* __restrict__ idx) {
  constexpr int KS = D / 16;  // MFMA k-steps over the head dim
  const int lane = threadIdx.x & 63, n = lane & 31, hf = lane >> 5;
  const int G = hq / hkv, g = k.h / G;
  const int t = k.t0 + lane;  // the row this lane ranks and writes
  const bool valid = t < k.T;
  const int c = valid ? t / block : 0;
  const int KH = topk - 1;
  int32_t* row = idx + (k.lrow + (valid ? t : 0)) * topk;

  const uint32_t mask = (1u << nbits) - 1u;
  uint32_t L[KHMAX];
#pragma unroll
  for (int p = 0; p < KHMAX; ++p) L[p] = 0u;

  const int cmax = wave_max_i32(c);
  const int cmin = -wave_max_i32(valid ? -c : -0x7fffffff);
  const size_t cbase = (size_t)(k.b * hkv + g) * nb;
  // ONE (nb <= 32): a single tile, so the query operands are dead after its MFMAs
  for (int jt = 0; ONE ? jt < 1 : jt * 32 < cmax; ++jt) {
    const int jrow = min(jt * 32 + n, nb - 1);
    const uint16_t* ph = chi + (cbase + jrow) * D + 8 * hf;
    const uint16_t* pl = clo + (cbase + jrow) * D + 8 * hf;
    const char* lh = lds + jrow * CentLds<D>::CS + 16 * hf;
    const char* ll = lh + nb * CentLds<D>::CS;
    f32x16_t acc0, acc1;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc0[i] = acc1[i] = 0.f;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const bf16x8_t ah = as_bf16x8(CLDS ? *reinterpret_cast<const u32x4_t*>(lh + 32 * s)
                                         : *reinterpret_cast<const u32x4_t*>(ph + 16 * s));
      const bf16x8_t al = as_bf16x8(CLDS ? *reinterpret_cast<const u32x4_t*>(ll + 32 * s)
                                         : *reinterpret_cast<const u32x4_t*>(pl + 16 * s));
      acc0 = mfma32x32x16(ah, bq[0][s], acc0);
      acc1 = mfma32x32x16(ah, bq[1][s], acc1);
      acc0 = mfma32x32x16(al, bq[0][s], acc0);
      acc1 = mfma32x32x16(al, bq[1][s], acc1);
    }
    // Lane halves swap: lane l < 32 keeps tile 0's scores of query l and receives the
    // other half of them from lane l + 32; lane l >= 32 receives tile 1's first half of
    // query l from lane l - 32 and keeps the second.  A[i] then holds block
    // (i/4)*8 + i%4 and B[i] block (i/4)*8 + 4 + i%4 of this tile, for query t0 + lane.
    uint32_t A[16], B[16];
    // a tile below every lane's current block needs no causal mask
    const bool full = (jt + 1) * 32 <= cmin;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc0[i]),
                                                      __float_as_uint(acc1[i]), false, false);
      const int ja = jt * 32 + (i >> 2) * 8 + (i & 3), jb = ja + 4;
      A[i] = gate_key(__uint_as_float(r[0]), mask - ja, mask);
      B[i] = gate_key(__uint_as_float(r[1]), mask - jb, mask);
    }
    if (!full) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int ja = jt * 32 + (i >> 2) * 8 + (i & 3), jb = ja + 4;
        A[i] = ja < c ? A[i] : 0u;
        B[i] = jb < c ? B[i] : 0u;
      }
    }
    sort16_desc(A);
    sort16_desc(B);
    if (KHMAX == 16) {
      // top 16 of the tile: A descending + B reversed is bitonic after the max
#pragma unroll
      for (int p = 0; p < 16; ++p) A[p] = max(A[p], B[15 - p]);
      bitonic_merge_desc(A);
      if (jt == 0) {
#pragma unroll
        for (int p = 0; p < 16; ++p) L[KHMAX - 16 + p] = A[p];
        continue;
      }
#pragma unroll
      for (int p = 0; p < 16; ++p) L[KHMAX - 16 + p] = max(L[KHMAX - 16 + p], A[15 - p]);
    } else {
      // all 32 keys of the tile, sorted: merge A and reversed B (a bitonic sequence)
      uint32_t M[32];
#pragma unroll
      for (int p = 0; p < 16; ++p) {
        M[p] = A[p];
        M[16 + p] = B[15 - p];
      }
      bitonic_merge_desc(M);
      if (jt == 0) {
        // the first tile's keys, sorted, head the list; the rest of a longer list stays
        // empty (0 ranks below every key), so the list is sorted for the merges below
#pragma unroll
        for (int p = 0; p < 32; ++p) L[p] = M[p];
        continue;
      }
#pragma unroll
      for (int p = 0; p < 32; ++p) L[KHMAX - 32 + p] = max(L[KHMAX - 32 + p], M[31 - p]);
    }
    // running list (descending) + reversed sorted tile list -> bitonic -> sorted
    bitonic_merge_desc(L);
  }

  if (!valid) return;
  // the best KH keys -> block ids, ascending
  int J[KHMAX];
  if (nb <= 32) {
    // a bit per selected block, then the set bits from the lowest up
    uint32_t sel = 0u;
#pragma unroll
    for (int p = 0; p < KHMAX; ++p)
      if (p < KH && L[p] != 0u) sel |= 1u << (mask - (L[p] & mask));
#pragma unroll
    for (int p = 0; p < KHMAX; ++p) {
      J[p] = (int)__builtin_ctz(sel | 0x80000000u);
      sel &= sel - 1u;
    }
  } else {
    // empty slots sort last
#pragma unroll
    for (int p = 0; p < KHMAX; ++p) {
      const bool keep = p < KH && L[p] != 0u;
      J[p] = keep ? (int)(mask - (L[p] & mask)) : 0x7fffffff;
    }
    bitonic_sort_asc(J);
  }
  const int nh = min(c, KH);
  // the row: nh history blocks ascending, the current block, then -1
  if ((topk & 3) == 0) {
#pragma unroll
    for (int p4 = 0; p4 * 4 <= KHMAX; ++p4) {
      if (p4 * 4 < topk) {
        int v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int p = p4 * 4 + e;
          v[e] = p < nh ? J[p < KHMAX ? p : 0] : (p == nh ? c : -1);
        }
        *reinterpret_cast<int4*>(row + p4 * 4) = make_int4(v[0], v[1], v[2], v[3]);
      }
    }
  } else {
#pragma unroll
    for (int p = 0; p <= KHMAX; ++p)
      if (p < topk) row[p] = p < nh ? J[p < KHMAX ? p : 0] : (p == nh ? c : -1);
  }
}

// KHMAX: list length (16, 32 or 64) >= topk-1.  D: head_dim.  One wavefront per chunk.
// Three wavefronts per SIMD: the loads of one chunk hide behind the ranking of others;
// the 64-long list needs the registers of two, and the single-tile LDS kernel (ONE)
// with the 16-long list fits four.
template <int KHMAX, bool ONE = false>
struct GateWaves {
  static constexpr int value = KHMAX > 32 ? 2 : (ONE && KHMAX == 16 ? 4 : 3);
};

template <int D, int KHMAX>
__global__ __launch_bounds__(kThreads, GateWaves<KHMAX>::value) void gate_topk_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ chi,
    const uint16_t* __restrict__ clo, int batch, SeqMap sq, int hq, int hkv, int block,
    int nb, int topk, int nbits, int32_t* __restrict__ idx) {
  const int nct = (sq.T + 63) / 64;
  const int nchunks = batch * hq * nct;
  const int cid = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (cid >= nchunks) return;
  const GateChunk k = gate_chunk_make(sq, cid / (nct * hq), (cid / nct) % hq,
                                      (cid % nct) * 64, hq, block, topk - 1);
  if (k.t0 >= k.T) return;   // past the end of a shorter packed sequence
  if (!k.compete) {
    gate_all_blocks(k, block, topk, idx);
    return;
  }
  bf16x8_t bq[2][D / 16];
  gate_load_q<D>(bq, q, k.T, hq, k.tok0, k.h, k.t0, true);
  gate_chunk<D, KHMAX, false>(bq, k, chi, clo, nullptr, hq, hkv, block, nb, topk, nbits,
                              idx);
}

// The same with the centroids in LDS (nb <= CentLds::MAX_NB): a workgroup takes four
// chunks of one (batch, kv-head) group, blockIdx.y = b * hkv + g, and first copies that
// kv-head's hi/lo centroids into LDS.
// ONE: nb <= 32, one tile of blocks: the LDS image is sized for 32 rows and, with the
// 16-long list, the kernel fits four wavefronts per SIMD (more query loads in flight).
template <int D, int KHMAX, bool ONE>
__global__ __launch_bounds__(kThreads, (GateWaves<KHMAX, ONE>::value))
void gate_topk_lds_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ chi,
    const uint16_t* __restrict__ clo, int batch, SeqMap sq, int hq, int hkv, int block,
    int nb, int topk, int nbits, int32_t* __restrict__ idx) {
  using CL = CentLds<D>;
  __shared__ __attribute__((aligned(16))) char lds[ONE ? 2 * 32 * CL::CS : CL::BYTES];
  const int G = hq / hkv, nct = (sq.T + 63) / 64;
  const int b = blockIdx.y / hkv, g = blockIdx.y % hkv;
  const int ci = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);   // chunk in group
  const size_t cbase = (size_t)(b * hkv + g) * nb;
  constexpr int CPR = D / 8;  // 16-byte chunks per centroid row
  for (int e = threadIdx.x; e < 2 * nb * CPR; e += kThreads) {
    const int which = e / (nb * CPR), r = (e / CPR) % nb, cp = e % CPR;
    const uint16_t* src = (which ? clo : chi) + (cbase + r) * D + cp * 8;
    *reinterpret_cast<u32x4_t*>(lds + (which * nb + r) * CL::CS + cp * 16) =
        *reinterpret_cast<const u32x4_t*>(src);
  }
  __syncthreads();
  if (ci >= G * nct) return;
  const GateChunk k = gate_chunk_make(sq, b, g * G + ci / nct, (ci % nct) * 64, hq, block,
                                      topk - 1);
  if (k.t0 >= k.T) return;   // past the end of a shorter packed sequence
  if (!k.compete) {
    gate_all_blocks(k, block, topk, idx);
    return;
  }
  bf16x8_t bq[2][D / 16];
  gate_load_q<D>(bq, q, k.T, hq, k.tok0, k.h, k.t0, true);
  gate_chunk<D, KHMAX, true, ONE>(bq, k, chi, clo, lds, hq, hkv, block, nb, topk, nbits,
                                  idx);
}

hipError_t launch_gate(const Shape& s, const uint16_t* q, const uint16_t* chi,
                       const uint16_t* clo, int32_t* idx, hipStream_t st) {
  const int nb = s.nb();
  int nbits = 1;
  while ((1 << nbits) < nb) ++nbits;
  // a wavefront per 64-token chunk of one query head
  const long nchunks = (long)s.b * s.hq * ((s.T + 63) / 64);
  const int per_block = kThreads / 64;
  dim3 grid((unsigned)((nchunks + per_block - 1) / per_block));
  const int KH = s.KH();
  const bool clds = nb <= 96;
  const long group_chunks = (long)s.G() * ((s.T + 63) / 64);
  const dim3 grid_lds((unsigned)((group_chunks + per_block - 1) / per_block), s.b * s.hkv);
#define MOBA_GATE(DD, KK)                                                                \
  do {                                                                                   \
    if (clds && nb <= 32)                                                                \
      hipLaunchKernelGGL((gate_topk_lds_kernel<DD, KK, true>), grid_lds, dim3(kThreads), 0, \
                         st, q, chi, clo, s.b, s.seqs(), s.hq, s.hkv, s.block, nb, s.topk, \
                         nbits, idx);                                                    \
    else if (clds)                                                                       \
      hipLaunchKernelGGL((gate_topk_lds_kernel<DD, KK, false>), grid_lds, dim3(kThreads), 0, \
                         st, q, chi, clo, s.b, s.seqs(), s.hq, s.hkv, s.block, nb, s.topk, \
                         nbits, idx);                                                    \
    else                                                                                 \
      hipLaunchKernelGGL((gate_topk_kernel<DD, KK>), grid, dim3(kThreads), 0, st, q, chi, \
                         clo, s.b, s.seqs(), s.hq, s.hkv, s.block, nb, s.topk, nbits,     \
                         idx);                                                           \
  } while (0)
  if (s.d == 128) {
    if (KH <= 16) MOBA_GATE(128, 16);
    else if (KH <= 32) MOBA_GATE(128, 32);
    else MOBA_GATE(128, 64);
  } else {
    if (KH <= 16) MOBA_GATE(64, 16);
    else if (KH <= 32) MOBA_GATE(64, 32);
    else MOBA_GATE(64, 64);
  }
#undef MOBA_GATE
  return hipGetLastError();
}

int gate_max_history() { return 64; }

// Rows of every (sequence, query head, token) when every causal block is selected:
// blocks 0 .. c ascending, then -1 (README bullet "Seamlessly Transition between Full
// and Sparse Attention": with every block selected, MoBA is full attention).
__global__ __launch_bounds__(kThreads) void idx_all_blocks_kernel(SeqMap sq, int hq,
                                                                  int block, int topk,
                                                                  int32_t* __restrict__ idx) {
  const int t = blockIdx.x * kThreads + threadIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
  if (t >= sq.len(b)) return;
  const int c = t / block;
  int32_t* row = idx + (sq.lrow(b, h, hq) + t) * topk;
  for (int p = 0; p < topk; ++p) row[p] = p <= c ? p : -1;
}

hipError_t launch_idx_all_blocks(const Shape& s, int32_t* idx, hipStream_t st) {
  hipLaunchKernelGGL(idx_all_blocks_kernel, dim3((s.T + kThreads - 1) / kThreads, s.hq, s.b),
                     dim3(kThreads), 0, st, s.seqs(), s.hq, s.block, s.topk, idx);
  return hipGetLastError();
}

}  // namespace moba
