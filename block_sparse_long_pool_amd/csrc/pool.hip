// Centroid mean-pool: C[b][g][j][:] = mean of the keys of block j of kv-head g of
// sequence b
// ("MoBA: Mixture of Block Attention for Long-Context LLMs", paper summary page,
// section "Approach": a block is represented by its mean-pooled key).
//
// HBM-bound.  When (sequence, block, kv-head) triples fill the chip (at least 256),
// one workgroup pools one block of one kv-head in a single pass: d/8 threads read a
// key row's d columns with 16-byte loads, sixteen rows in flight per thread, and the
// per-thread float32 sums are added in a fixed order in LDS (deterministic, no
// atomics).  Otherwise a token's keys for all kv-heads, one contiguous row of hkv*d
// bf16, are read by workgroups over `splits` token ranges of each block, and a second
// pass adds the split partials in a fixed order and divides by the token count.
#include "moba_internal.h"

namespace moba {

// c -> bf16 hi + bf16 lo, c ~= hi + lo to ~2^-17 relative (c - hi is exact in fp32)
__device__ __forceinline__ void split_hi_lo(float c, uint16_t* hi_out, uint16_t* lo_out) {
  const uint32_t hi = f32_to_bf16_rne(c);
  *hi_out = (uint16_t)hi;
  *lo_out = (uint16_t)f32_to_bf16_rne(c - __uint_as_float(hi << 16));
}

__global__ __launch_bounds__(kThreads) void pool_partial_kernel(
    const uint16_t* __restrict__ k, SeqMap sq, int cols, int block, int rows_per_split,
    float* __restrict__ partial) {
  const int s = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  const int T = sq.len(b), tok0 = sq.tok0(b);
  const int splits = gridDim.x, nb = gridDim.y;
  const int W = cols / 8;                    // 16-byte column chunks per row
  const int R = W >= kThreads ? 1 : kThreads / W;
  const int tid = threadIdx.x;
  const int rsub = W >= kThreads ? 0 : tid / W;
  const int cstart = W >= kThreads ? tid : tid % W;
  const int cstep = W >= kThreads ? kThreads : W;
  const int row0 = j * block + s * rows_per_split;
  const int row1 = min(min(row0 + rows_per_split, (j + 1) * block), T);
  __shared__ float red[2048];                // R * cols <= 2048 whenever R > 1
  float* dst = partial + ((size_t)(b * nb + j) * splits + s) * cols;

  for (int cc = cstart; cc < W; cc += cstep) {
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    if (rsub < R) {
      const uint16_t* p = k + ((size_t)tok0 + row0 + rsub) * cols + cc * 8;
      const size_t stride = (size_t)R * cols;
      for (int row = row0 + rsub; row < row1; row += R, p += stride) {
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(p);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] += bf16lo(v[e]);
          acc[2 * e + 1] += bf16hi(v[e]);
        }
      }
    }
    if (R == 1) {
#pragma unroll
      for (int e = 0; e < 8; ++e) dst[cc * 8 + e] = acc[e];
    } else if (rsub < R) {
#pragma unroll
      for (int e = 0; e < 8; ++e) red[rsub * cols + cc * 8 + e] = acc[e];
    }
  }
  if (R > 1) {
    __syncthreads();
    for (int c = tid; c < cols; c += kThreads) {
      float sum = 0.f;
      for (int r = 0; r < R; ++r) sum += red[r * cols + c];
      dst[c] = sum;
    }
  }
}

// sum the split partials in order, divide by the block's token count (a block past
// the end of a shorter packed sequence gets 0; no query ever scores it); with chi/clo,
// also the bf16 hi + lo split the gate reads (c ~= hi + lo to ~2^-17 relative)
__global__ __launch_bounds__(kThreads) void pool_finalize_kernel(
    const float* __restrict__ partial, int b_, SeqMap sq, int hkv, int d, int block, int nb,
    int splits, float* __restrict__ cent, uint16_t* __restrict__ chi,
    uint16_t* __restrict__ clo) {
  const size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  const size_t total = (size_t)b_ * hkv * nb * d;
  if (i >= total) return;
  const int dim = (int)(i % d);
  const int j = (int)((i / d) % nb);
  const int g = (int)((i / ((size_t)d * nb)) % hkv);
  const int b = (int)(i / ((size_t)d * nb * hkv));
  const int cols = hkv * d;
  const float* p = partial + ((size_t)(b * nb + j) * splits) * cols + g * d + dim;
  float sum = 0.f;
  for (int s = 0; s < splits; ++s) sum += p[(size_t)s * cols];
  const int n = min(block, sq.len(b) - j * block);
  const float c = n > 0 ? sum / (float)n : 0.f;
  cent[i] = c;  // layout [b][hkv][nb][d] == i
  if (chi != nullptr) split_hi_lo(c, chi + i, clo + i);
}

// one block j of kv-head g of sequence b, in one pass (the layout of cent, chi, clo is
// [b][hkv][nb][d]); a block past the end of a shorter packed sequence gets 0
template <int D>
__global__ __launch_bounds__(kThreads) void pool_block_kernel(
    const uint16_t* __restrict__ k, SeqMap sq, int hkv, int block, int nb,
    float* __restrict__ cent, uint16_t* __restrict__ chi, uint16_t* __restrict__ clo) {
  constexpr int CPR = D / 8;                 // 16-byte chunks per key row
  constexpr int RP = kThreads / CPR;         // rows per pass
  constexpr int U = 16;                      // rows in flight per thread
  __shared__ float red[RP * D];
  const int g = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  const int T = sq.len(b), tok0 = sq.tok0(b);
  const int row0 = j * block, row1 = min((j + 1) * block, T);
  const int tid = threadIdx.x, rsub = tid / CPR, cc = tid % CPR;
  const size_t rs = (size_t)hkv * D;         // elements from one token's keys to the next
  const uint16_t* base = k + ((size_t)tok0 * hkv + g) * D + cc * 8;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  auto add = [&](const u32x4_t& v) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] += bf16lo(v[e]);
      acc[2 * e + 1] += bf16hi(v[e]);
    }
  };
  int row = row0 + rsub;
  for (; row + (U - 1) * RP < row1; row += U * RP) {
    u32x4_t v[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      v[u] = *reinterpret_cast<const u32x4_t*>(base + (size_t)(row + u * RP) * rs);
#pragma unroll
    for (int u = 0; u < U; ++u) add(v[u]);
  }
  for (; row < row1; row += RP) add(*reinterpret_cast<const u32x4_t*>(base + (size_t)row * rs));
#pragma unroll
  for (int e = 0; e < 8; ++e) red[rsub * D + cc * 8 + e] = acc[e];
  __syncthreads();
  if (tid < D) {
    float sum = 0.f;
    for (int r = 0; r < RP; ++r) sum += red[r * D + tid];
    const int n = row1 - row0;
    const float c = n > 0 ? sum / (float)n : 0.f;
    const size_t i = (((size_t)b * hkv + g) * nb + j) * D + tid;
    cent[i] = c;
    if (chi != nullptr) split_hi_lo(c, chi + i, clo + i);
  }
}

__global__ __launch_bounds__(kThreads) void centroid_split_kernel(
    const float* __restrict__ cent, size_t total, uint16_t* __restrict__ chi,
    uint16_t* __restrict__ clo) {
  const size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= total) return;
  split_hi_lo(cent[i], chi + i, clo + i);
}

int pool_splits(const Shape& s) {
  const int nb = s.nb();
  int splits = (2048 + s.b * nb - 1) / (s.b * nb);
  splits = max(1, min(splits, s.block / 16));
  return splits;
}

hipError_t launch_pool(const Shape& s, const uint16_t* k, float* partial, float* cent,
                       uint16_t* chi, uint16_t* clo, hipStream_t st) {
  const int nb = s.nb();
  if ((long)s.b * nb * s.hkv >= 256) {
    const dim3 grid(s.hkv, nb, s.b);
    if (s.d == 128)
      hipLaunchKernelGGL(pool_block_kernel<128>, grid, dim3(kThreads), 0, st, k, s.seqs(),
                         s.hkv, s.block, nb, cent, chi, clo);
    else
      hipLaunchKernelGGL(pool_block_kernel<64>, grid, dim3(kThreads), 0, st, k, s.seqs(),
                         s.hkv, s.block, nb, cent, chi, clo);
    return hipGetLastError();
  }
  const int splits = pool_splits(s);
  const int rows_per_split = (s.block + splits - 1) / splits;
  const int cols = s.hkv * s.d;
  dim3 grid(splits, nb, s.b);
  hipLaunchKernelGGL(pool_partial_kernel, grid, dim3(kThreads), 0, st, k, s.seqs(), cols,
                     s.block, rows_per_split, partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t total = (size_t)s.b * s.hkv * nb * s.d;
  hipLaunchKernelGGL(pool_finalize_kernel, dim3((unsigned)((total + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, st, partial, s.b, s.seqs(), s.hkv, s.d, s.block, nb,
                     splits, cent, chi, clo);
  return hipGetLastError();
}

hipError_t launch_centroid_split(const Shape& s, const float* cent, uint16_t* chi,
                                 uint16_t* clo, hipStream_t st) {
  const size_t total = (size_t)s.b * s.hkv * s.nb() * s.d;
  hipLaunchKernelGGL(centroid_split_kernel,
                     dim3((unsigned)((total + kThreads - 1) / kThreads)), dim3(kThreads),
                     0, st, cent, total, chi, clo);
  return hipGetLastError();
}

}  // namespace moba
