// Inverted index: for every KV block, the list of query rows that selected it as a
// history block.  This is the "gather" half of Gather-and-Densify in the FlashMoBA
// story (hyper.ai, paragraph on Gather-and-Densify): the queries scattered over the
// sequence that chose one block are collected so the attention kernel can run them
// as one dense tile against that block.
//
// Rows of kv-head g are r = t*G + h%G.  Rows are cut into chunks of 256 (one
// workgroup).  Pass 1 counts, per chunk, how many rows chose each block (LDS
// atomics; counts are order-free).  Pass 2 turns the counts into per-chunk bases by
// an exclusive scan over chunks, and the list totals into list offsets and a tile
// list.  Pass 3 writes the entries: for each history slot in turn, a wavefront finds
// the lanes holding the same block with one ballot per bit of the block id
// (multi-split), ranks them with a popcount, and combines the four wavefronts through
// LDS.  The order inside a list is therefore (chunk, slot, row): deterministic.
#include "moba_internal.h"

namespace moba {

constexpr int kChunk = 256;  // rows per chunk == threads per workgroup

int index_chunks(const Shape& s) {
  const long rows = (long)s.T * s.G();
  return (int)((rows + kChunk - 1) / kChunk);
}

__global__ __launch_bounds__(kThreads) void index_count_kernel(
    const int32_t* __restrict__ idx, SeqMap sq, int hq, int G, int block, int topk, int nb,
    int g0, int ng, int nchunks, int32_t* __restrict__ chunk_counts) {
  extern __shared__ int32_t cnt[];
  const int chunk = blockIdx.x, gi = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  for (int j = tid; j < nb; j += kThreads) cnt[j] = 0;
  __syncthreads();
  const long r = (long)chunk * kChunk + tid;
  const int t = (int)(r / G), hl = (int)(r % G);
  if (t < sq.len(b)) {
    const int c = t / block;
    const int h = (g0 + gi) * G + hl;
    const int32_t* row = idx + (sq.lrow(b, h, hq) + t) * topk;
    for (int s = 0; s < topk - 1; ++s) {
      const int j = row[s];
      if (j >= 0 && j < c) atomicAdd(&cnt[j], 1);
    }
  }
  __syncthreads();
  int32_t* dst = chunk_counts + ((size_t)(b * ng + gi) * nchunks + chunk) * nb;
  for (int j = tid; j < nb; j += kThreads) dst[j] = cnt[j];
}

// exclusive scan over chunks of one list (b, gi, j), in place; total -> list_count
__global__ __launch_bounds__(kThreads) void index_scan_chunks_kernel(
    int32_t* __restrict__ chunk_counts, int nb, int ng, int nchunks,
    int32_t* __restrict__ list_count) {
  const int j = blockIdx.x, gi = blockIdx.y, b = blockIdx.z;
  int32_t* base = chunk_counts + (size_t)(b * ng + gi) * nchunks * nb + j;
  __shared__ int32_t sh[kThreads];
  __shared__ int32_t carry;
  if (threadIdx.x == 0) carry = 0;
  __syncthreads();
  for (int c0 = 0; c0 < nchunks; c0 += kThreads) {
    const int c = c0 + threadIdx.x;
    const int v = c < nchunks ? base[(size_t)c * nb] : 0;
    sh[threadIdx.x] = v;
    __syncthreads();
    // Hillis-Steele inclusive scan
    for (int o = 1; o < kThreads; o <<= 1) {
      const int x = threadIdx.x >= o ? sh[threadIdx.x - o] : 0;
      __syncthreads();
      sh[threadIdx.x] += x;
      __syncthreads();
    }
    const int incl = sh[threadIdx.x];
    const int cr = carry;
    if (c < nchunks) base[(size_t)c * nb] = cr + incl - v;
    __syncthreads();
    if (threadIdx.x == kThreads - 1) carry = cr + incl;
    __syncthreads();
  }
  if (threadIdx.x == 0) list_count[(b * ng + gi) * nb + j] = carry;
}

// one workgroup: list offsets and tile offsets (exclusive scans over all lists)
__global__ __launch_bounds__(kThreads) void index_scan_lists_kernel(
    const int32_t* __restrict__ list_count, int nlists, int tile_m,
    int32_t* __restrict__ list_offsets, int32_t* __restrict__ tile_offsets) {
  __shared__ int32_t sa[kThreads], sb[kThreads];
  __shared__ int32_t ca, cb;
  if (threadIdx.x == 0) { ca = 0; cb = 0; }
  __syncthreads();
  for (int l0 = 0; l0 < nlists; l0 += kThreads) {
    const int l = l0 + threadIdx.x;
    const int v = l < nlists ? list_count[l] : 0;
    const int w = (v + tile_m - 1) / tile_m;
    sa[threadIdx.x] = v;
    sb[threadIdx.x] = w;
    __syncthreads();
    for (int o = 1; o < kThreads; o <<= 1) {
      const int x = threadIdx.x >= o ? sa[threadIdx.x - o] : 0;
      const int y = threadIdx.x >= o ? sb[threadIdx.x - o] : 0;
      __syncthreads();
      sa[threadIdx.x] += x;
      sb[threadIdx.x] += y;
      __syncthreads();
    }
    const int ia = sa[threadIdx.x], ib = sb[threadIdx.x];
    const int a0 = ca, b0 = cb;
    if (l < nlists) {
      list_offsets[l] = a0 + ia - v;
      tile_offsets[l] = b0 + ib - w;
    }
    __syncthreads();
    if (threadIdx.x == kThreads - 1) { ca = a0 + ia; cb = b0 + ib; }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    list_offsets[nlists] = ca;
    tile_offsets[nlists] = cb;  // number of tiles
  }
}

// tiles[i] = {list, begin, end, 0}
__global__ __launch_bounds__(64) void index_tiles_kernel(
    const int32_t* __restrict__ list_offsets, const int32_t* __restrict__ tile_offsets,
    int tile_m, int4* __restrict__ tiles) {
  const int l = blockIdx.x;
  const int b0 = list_offsets[l], b1 = list_offsets[l + 1];
  const int t0 = tile_offsets[l];
  const int nt = tile_offsets[l + 1] - t0;
  for (int i = threadIdx.x; i < nt; i += 64) {
    const int s = b0 + i * tile_m;
    tiles[t0 + i] = make_int4(l, s, min(s + tile_m, b1), 0);
  }
}

__global__ __launch_bounds__(kThreads) void index_scatter_kernel(
    const int32_t* __restrict__ idx, SeqMap sq, int hq, int G, int block, int topk, int nb,
    int nbits, int g0, int ng, int nchunks, const int32_t* __restrict__ chunk_base,
    const int32_t* __restrict__ list_offsets, uint32_t* __restrict__ entries,
    long long cap) {
  extern __shared__ int32_t lds[];
  int32_t* base = lds;            // [nb]  absolute start of this chunk's part of list j
  int32_t* run = lds + nb;        // [nb]  entries of this chunk already placed
  int32_t* wcnt = lds + 2 * nb;   // [4][nb] per-wavefront counts of the current slot
  const int chunk = blockIdx.x, gi = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int list0 = (b * ng + gi) * nb;
  const int32_t* cb = chunk_base + ((size_t)(b * ng + gi) * nchunks + chunk) * nb;
  for (int j = tid; j < nb; j += kThreads) {
    base[j] = list_offsets[list0 + j] + cb[j];
    run[j] = 0;
    wcnt[j] = wcnt[nb + j] = wcnt[2 * nb + j] = wcnt[3 * nb + j] = 0;
  }
  __syncthreads();
  const long r = (long)chunk * kChunk + tid;
  const int t = (int)(r / G), hl = (int)(r % G);
  const bool valid = t < sq.len(b);
  const int c = valid ? t / block : 0;
  const int32_t* row = idx + (sq.lrow(b, (g0 + gi) * G + hl, hq) + (valid ? t : 0)) * topk;
  const uint64_t below = (1ull << lane) - 1ull;
  for (int s = 0; s < topk - 1; ++s) {
    int j = valid ? row[s] : -1;
    const bool has = j >= 0 && j < c;
    if (!has) j = 0;
    uint64_t peers = __ballot(has);
    for (int bit = 0; bit < nbits; ++bit) {
      const bool on = (j >> bit) & 1;
      const uint64_t m = __ballot(has && on);
      peers &= on ? m : ~m;
    }
    const int rank = __popcll(peers & below);
    const bool leader = has && rank == 0;
    if (leader) wcnt[wave * nb + j] = __popcll(peers);
    __syncthreads();
    int before = 0;
    if (has) {
      for (int w = 0; w < wave; ++w) before += wcnt[w * nb + j];
      const int pos = base[j] + run[j] + before + rank;
      // a well-formed idx never reaches cap; a malformed one must not write past it
      if (pos < cap) entries[pos] = ((uint32_t)(t * G + hl) << 5) | (uint32_t)s;
    }
    __syncthreads();
    if (leader && before == 0) {
      run[j] += wcnt[j] + wcnt[nb + j] + wcnt[2 * nb + j] + wcnt[3 * nb + j];
    }
    __syncthreads();
    if (leader) wcnt[wave * nb + j] = 0;
    __syncthreads();
  }
}

hipError_t launch_index(const Shape& s, const int32_t* idx, int g0, int ng, int tile_m,
                        int32_t* chunk_counts, int32_t* list_count,
                        int32_t* list_offsets, int32_t* tile_offsets, int4* tiles,
                        uint32_t* entries, long long cap, hipStream_t st) {
  const int nb = s.nb();
  const int nchunks = index_chunks(s);
  int nbits = 1;
  while ((1 << nbits) < nb) ++nbits;
  const int nlists = s.b * ng * nb;
  dim3 grid(nchunks, ng, s.b);
  hipLaunchKernelGGL(index_count_kernel, grid, dim3(kThreads), nb * sizeof(int32_t), st,
                     idx, s.seqs(), s.hq, s.G(), s.block, s.topk, nb, g0, ng, nchunks,
                     chunk_counts);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(index_scan_chunks_kernel, dim3(nb, ng, s.b), dim3(kThreads), 0, st,
                     chunk_counts, nb, ng, nchunks, list_count);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(index_scan_lists_kernel, dim3(1), dim3(kThreads), 0, st, list_count,
                     nlists, tile_m, list_offsets, tile_offsets);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (tiles != nullptr) {
    hipLaunchKernelGGL(index_tiles_kernel, dim3(nlists), dim3(64), 0, st, list_offsets,
                       tile_offsets, tile_m, tiles);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(index_scatter_kernel, grid, dim3(kThreads), 6 * nb * sizeof(int32_t),
                     st, idx, s.seqs(), s.hq, s.G(), s.block, s.topk, nb, nbits, g0, ng,
                     nchunks, chunk_counts, list_offsets, entries, cap);
  return hipGetLastError();
}

}  // namespace moba
