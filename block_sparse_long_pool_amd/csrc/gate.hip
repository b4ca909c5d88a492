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
// Mapping.  A wavefront owns 32 query rows r = t*G + h%G of one kv-head g and
// computes S^T = C Q^T on MFMA 32x32x16 (rows = 32 blocks, columns = 32 queries).
// The centroid is float32; it enters the MFMA as bf16 hi + bf16 lo (two products
// into one float32 accumulator), the query is bf16 already.  Lane l then holds 16
// scores of query l%32 (blocks (i/4)*8 + (l/32)*4 + i%4).
//
// Ranking.  Each score becomes a 32-bit key whose high bits order like the float and
// whose low nbits hold (mask - j), so larger key = better, and exactly equal scores
// rank the lower block first.  Scores closer than ~2^-(23-nbits) relative compare
// as equal (well inside the 1e-3-relative near-tie band).  Each lane sorts its 16
// keys with a bitonic network and merges them into a running sorted top-KHMAX list;
// the two lanes of a query merge their lists at the end.  No branch depends on the
// data, so the wavefront never diverges.
#include "moba_internal.h"

namespace moba {

namespace {

__device__ __forceinline__ uint32_t gate_key(float s, int j, uint32_t mask) {
  uint32_t u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0u;  // -0 ranks like +0
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (u & ~mask) | (mask - (uint32_t)j);
}

template <int N>
__device__ __forceinline__ void cas_desc(uint32_t (&a)[N], int i, int k) {
  const uint32_t x = a[i], y = a[k];
  a[i] = max(x, y);
  a[k] = min(x, y);
}

// full bitonic sort, descending
template <int N>
__device__ __forceinline__ void bitonic_sort_desc(uint32_t (&a)[N]) {
#pragma unroll
  for (int kk = 2; kk <= N; kk <<= 1) {
#pragma unroll
    for (int jj = kk >> 1; jj > 0; jj >>= 1) {
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const int ixj = i ^ jj;
        if (ixj > i) {
          if ((i & kk) == 0) cas_desc(a, i, ixj);
          else cas_desc(a, ixj, i);
        }
      }
    }
  }
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

// KHMAX: list length (16 or 32) >= topk-1.  D: head_dim.
template <int D, int KHMAX>
__global__ __launch_bounds__(kThreads) void gate_topk_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ chi,
    const uint16_t* __restrict__ clo, int T, int hq, int hkv, int block, int nb,
    int topk, int nbits, int32_t* __restrict__ idx) {
  constexpr int KS = D / 16;  // MFMA k-steps over the head dim
  const int G = hq / hkv;
  const int b = blockIdx.z, g = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 31, hf = lane >> 5;
  const int r = (blockIdx.x * 4 + wave) * 32 + n;
  const int t = r / G, hl = r % G, h = g * G + hl;
  const bool valid = t < T;
  const int c = valid ? t / block : 0;
  const int KH = topk - 1;
  // does any row of this wavefront have more candidates than slots?
  const bool compete = valid && c > KH;
  const bool wave_compete = __ballot(compete) != 0ull;

  int32_t* row = idx + ((size_t)(b * hq + h) * T + (valid ? t : 0)) * topk;

  if (!wave_compete) {
    // every causal block is selected: 0..c, then -1
    if (valid && hf == 0) {
      for (int p = 0; p < topk; ++p) row[p] = p <= c ? p : -1;
    }
    return;
  }

  // query operand: dims 16*s + 8*hf .. +7 of row (t, h)
  bf16x8_t bq[KS];
  {
    const uint16_t* qp = q + ((size_t)((size_t)b * T + (valid ? t : 0)) * hq + h) * D + 8 * hf;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      u32x4_t v = *reinterpret_cast<const u32x4_t*>(qp + 16 * s);
      if (!valid) v = u32x4_t{0u, 0u, 0u, 0u};
      bq[s] = as_bf16x8(v);
    }
  }
  const uint32_t mask = (1u << nbits) - 1u;
  uint32_t L[KHMAX];
#pragma unroll
  for (int p = 0; p < KHMAX; ++p) L[p] = 0u;

  const int cmax = wave_max_i32(c);
  const size_t cbase = (size_t)(b * hkv + g) * nb;
  for (int jt = 0; jt * 32 < cmax; ++jt) {
    const int jrow = min(jt * 32 + n, nb - 1);
    const uint16_t* ph = chi + (cbase + jrow) * D + 8 * hf;
    const uint16_t* pl = clo + (cbase + jrow) * D + 8 * hf;
    f32x16_t acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const bf16x8_t ah = as_bf16x8(*reinterpret_cast<const u32x4_t*>(ph + 16 * s));
      const bf16x8_t al = as_bf16x8(*reinterpret_cast<const u32x4_t*>(pl + 16 * s));
      acc = mfma32x32x16(ah, bq[s], acc);
      acc = mfma32x32x16(al, bq[s], acc);
    }
    uint32_t N16[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int j = jt * 32 + (i >> 2) * 8 + hf * 4 + (i & 3);
      N16[i] = (j < c) ? gate_key(acc[i], j, mask) : 0u;
    }
    bitonic_sort_desc(N16);
    // running list (descending) + reversed new sorted run -> bitonic top-KHMAX
#pragma unroll
    for (int p = KHMAX - 16; p < KHMAX; ++p) L[p] = max(L[p], N16[KHMAX - 1 - p]);
    bitonic_merge_desc(L);
  }
  // merge with the other half of the query's blocks (lane ^ 32)
#pragma unroll
  for (int p = 0; p < KHMAX; ++p) {
    const uint32_t other = xor32_u32(L[KHMAX - 1 - p]);
    L[p] = max(L[p], other);
  }
  bitonic_merge_desc(L);

  if (!valid) return;
  // the best KH keys -> block ids, ascending; empty slots sort last
  int J[KHMAX];
#pragma unroll
  for (int p = 0; p < KHMAX; ++p) {
    const bool keep = p < KH && L[p] != 0u;
    J[p] = keep ? (int)(mask - (L[p] & mask)) : 0x7fffffff;
  }
  bitonic_sort_asc(J);
  const int nh = min(c, KH);
  // lanes hf = 0 / 1 write the first / second half of the row
  const int half = (topk + 1) >> 1;
  const int p0 = hf ? half : 0, p1 = hf ? topk : half;
#pragma unroll
  for (int p = 0; p <= KHMAX; ++p) {
    if (p >= p0 && p < p1) {
      int val;
      if (p < nh) val = J[p < KHMAX ? p : 0];
      else val = (p == nh) ? c : -1;
      row[p] = val;
    }
  }
}

hipError_t launch_gate(const Shape& s, const uint16_t* q, const uint16_t* chi,
                       const uint16_t* clo, int32_t* idx, hipStream_t st) {
  const int nb = s.nb();
  int nbits = 1;
  while ((1 << nbits) < nb) ++nbits;
  const long rows = (long)s.T * s.G();
  dim3 grid((unsigned)((rows + 127) / 128), s.hkv, s.b);
  const int KH = s.KH();
#define MOBA_GATE(DD, KK)                                                            \
  hipLaunchKernelGGL((gate_topk_kernel<DD, KK>), grid, dim3(kThreads), 0, st, q, chi, \
                     clo, s.T, s.hq, s.hkv, s.block, nb, s.topk, nbits, idx)
  if (s.d == 128) {
    if (KH <= 16) MOBA_GATE(128, 16);
    else MOBA_GATE(128, 32);
  } else {
    if (KH <= 16) MOBA_GATE(64, 16);
    else MOBA_GATE(64, 32);
  }
#undef MOBA_GATE
  return hipGetLastError();
}

}  // namespace moba
