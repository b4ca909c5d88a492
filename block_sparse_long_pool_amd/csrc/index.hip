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

// A row's history slots are counted and listed only where the block id first appears
// in the row.  A selection from the gate never repeats a block; a caller-built idx
// that does still yields at most min(c, k-1) entries per row, so the lists, tiles and
// entries stay within the sizes the host derives from the shape.  `above` is the
// largest id of slots 0 .. s-1: an id above it is new without a look back, which is
// every slot of an ascending row (the gate's order).
__device__ __forceinline__ bool first_in_row(const int32_t* __restrict__ row, int s, int j,
                                             int above) {
  if (j > above) return true;
  for (int u = 0; u < s; ++u)
    if (row[u] == j) return false;
  return true;
}

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
    int above = -1;
    for (int s = 0; s < topk - 1; ++s) {
      const int j = row[s];
      if (j >= 0 && j < c && first_in_row(row, s, j, above)) atomicAdd(&cnt[j], 1);
      above = max(above, j);
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
    tile_offsets[nlists + 1] = 0;  // the history kernel's tile queue starts empty
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

// One workgroup: one chunk of rows and one range of at most kRange blocks (its LDS
// tables hold 6 ints per block of the range); blockIdx.x = chunk + nchunks * range.
// The rows are read once per range, so block counts beyond kRange cost extra reads
// of idx but no more LDS.
//
// STAGED (a chunk has at most kStageEntries entries, the range at most kStageMaxRange
// blocks, and the launcher's rule below holds): the entries are placed in LDS first, each list's run of the
// chunk at its offset in the chunk (an exclusive scan of the chunk's list counts,
// which the chunk bases already hold), and then written out with consecutive lanes
// on consecutive positions of each run.  Written straight from the ranking, each
// slot's pass would store one 4-byte entry into most of the chunk's runs, so every
// run's cache line would be written once per slot; at 64K tokens with 128-key blocks
// those partial lines made the kernel fetch 1.5 GB to write 126 MB of entries.
constexpr int kRange = 2048;
constexpr int kStageEntries = 4096;
constexpr int kStageMaxRange = 1024;

template <bool STAGED>
__global__ __launch_bounds__(kThreads) void index_scatter_kernel(
    const int32_t* __restrict__ idx, SeqMap sq, int hq, int G, int block, int topk, int nb,
    int g0, int ng, int nchunks, const int32_t* __restrict__ chunk_base,
    const int32_t* __restrict__ list_count, const int32_t* __restrict__ list_offsets,
    uint32_t* __restrict__ entries, long long cap) {
  extern __shared__ int32_t lds[];
  __shared__ int32_t part[kThreads];
  __shared__ int32_t staged_total;
  const int chunk = blockIdx.x % nchunks, gi = blockIdx.y, b = blockIdx.z;
  const int j0 = (blockIdx.x / nchunks) * kRange;       // first block of the range
  const int nr = min(kRange, nb - j0);                   // blocks in the range
  int32_t* base = lds;            // [nr]  absolute start of this chunk's part of list j
  int32_t* run = lds + nr;        // [nr]  entries of this chunk already placed
  int32_t* wcnt = lds + 2 * nr;   // [4][nr] per-wavefront counts of the current slot
  int32_t* loff = lds + 6 * nr;   // [nr]  (STAGED) start of list j's run in the stage
  uint32_t* sval = reinterpret_cast<uint32_t*>(lds + 7 * nr);              // (STAGED)
  uint16_t* sid = reinterpret_cast<uint16_t*>(lds + 7 * nr + kStageEntries);  // (STAGED)
  int nbits = 1;
  while ((1 << nbits) < nr) ++nbits;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int list0 = (b * ng + gi) * nb + j0;
  const int32_t* cb = chunk_base + ((size_t)(b * ng + gi) * nchunks + chunk) * nb + j0;
  for (int j = tid; j < nr; j += kThreads) {
    base[j] = list_offsets[list0 + j] + cb[j];
    run[j] = 0;
    wcnt[j] = wcnt[nr + j] = wcnt[2 * nr + j] = wcnt[3 * nr + j] = 0;
    if (STAGED) {
      // the chunk's count of list j: the next chunk's base (or the list total) - this
      const int next = chunk + 1 < nchunks ? cb[nb + j] : list_count[list0 + j];
      loff[j] = next - cb[j];
    }
  }
  __syncthreads();
  if (STAGED) {
    // exclusive scan of the counts over the range: thread t owns ceil(nr / 256)
    // consecutive lists
    const int E = (nr + kThreads - 1) / kThreads;
    int v[kStageMaxRange / kThreads];
    int sum = 0;
#pragma unroll
    for (int e = 0; e < kStageMaxRange / kThreads; ++e) {
      const int j = tid * E + e;
      v[e] = (e < E && j < nr) ? loff[j] : 0;
      sum += v[e];
    }
    part[tid] = sum;
    __syncthreads();
    for (int o = 1; o < kThreads; o <<= 1) {
      const int x = tid >= o ? part[tid - o] : 0;
      __syncthreads();
      part[tid] += x;
      __syncthreads();
    }
    int at = part[tid] - sum;
#pragma unroll
    for (int e = 0; e < kStageMaxRange / kThreads; ++e) {
      const int j = tid * E + e;
      if (e < E && j < nr) {
        loff[j] = at;
        at += v[e];
      }
    }
    if (tid == kThreads - 1) staged_total = part[tid];
    __syncthreads();
  }
  const long r = (long)chunk * kChunk + tid;
  const int t = (int)(r / G), hl = (int)(r % G);
  const bool valid = t < sq.len(b);
  const int c = valid ? t / block : 0;
  const int32_t* row = idx + (sq.lrow(b, (g0 + gi) * G + hl, hq) + (valid ? t : 0)) * topk;
  const uint64_t below = (1ull << lane) - 1ull;
  const int sbits = entry_slot_bits(topk);
  int above = -1;
  for (int s = 0; s < topk - 1; ++s) {
    int j = valid ? row[s] : -1;
    const bool has = j >= j0 && j < j0 + nr && j < c && first_in_row(row, s, j, above);
    above = max(above, j);
    j = has ? j - j0 : 0;         // the block's place in the range
    uint64_t peers = __ballot(has);
    for (int bit = 0; bit < nbits; ++bit) {
      const bool on = (j >> bit) & 1;
      const uint64_t m = __ballot(has && on);
      peers &= on ? m : ~m;
    }
    const int rank = __popcll(peers & below);
    const bool leader = has && rank == 0;
    if (leader) wcnt[wave * nr + j] = __popcll(peers);
    __syncthreads();
    int before = 0;
    if (has) {
      for (int w = 0; w < wave; ++w) before += wcnt[w * nr + j];
      const uint32_t ent = ((uint32_t)(t * G + hl) << sbits) | (uint32_t)s;
      if (STAGED) {
        const int lp = loff[j] + run[j] + before + rank;
        if (lp < kStageEntries) {
          sval[lp] = ent;
          sid[lp] = (uint16_t)j;
        }
      } else {
        const int pos = base[j] + run[j] + before + rank;
        // a well-formed idx never reaches cap; a malformed one must not write past it
        if (pos < cap) entries[pos] = ent;
      }
    }
    __syncthreads();
    if (leader && before == 0) {
      run[j] += wcnt[j] + wcnt[nr + j] + wcnt[2 * nr + j] + wcnt[3 * nr + j];
    }
    __syncthreads();
    if (leader) wcnt[wave * nr + j] = 0;
    __syncthreads();
  }
  if (STAGED) {
    const int total = min(staged_total, kStageEntries);
    for (int i = tid; i < total; i += kThreads) {
      const int j = sid[i];
      const long long pos = (long long)base[j] + (i - loff[j]);
      if (pos < cap) entries[pos] = sval[i];
    }
  }
}

// tile_offsets of lists given by their offsets alone: the exclusive scan of
// ceil(count / tile_m) over lists, the total in tile_offsets[nlists] (one workgroup)
__global__ __launch_bounds__(kThreads) void tiles_scan_kernel(
    const int32_t* __restrict__ list_offsets, int nlists, int tile_m,
    int32_t* __restrict__ tile_offsets) {
  __shared__ int32_t sb[kThreads];
  __shared__ int32_t cb;
  if (threadIdx.x == 0) cb = 0;
  __syncthreads();
  for (int l0 = 0; l0 < nlists; l0 += kThreads) {
    const int l = l0 + threadIdx.x;
    const int w = l < nlists ? (list_offsets[l + 1] - list_offsets[l] + tile_m - 1) / tile_m : 0;
    sb[threadIdx.x] = w;
    __syncthreads();
    for (int o = 1; o < kThreads; o <<= 1) {
      const int y = threadIdx.x >= o ? sb[threadIdx.x - o] : 0;
      __syncthreads();
      sb[threadIdx.x] += y;
      __syncthreads();
    }
    const int ib = sb[threadIdx.x];
    const int b0 = cb;
    if (l < nlists) tile_offsets[l] = b0 + ib - w;
    __syncthreads();
    if (threadIdx.x == kThreads - 1) cb = b0 + ib;
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    tile_offsets[nlists] = cb;
    tile_offsets[nlists + 1] = 0;  // the history kernel's tile queue starts empty
  }
}

// dst[i] = src[(a * i + c) mod n] for the n tiles: a is the first number coprime to n
// at or after a seeded start, so the map is a permutation of the tile order
__global__ __launch_bounds__(256) void tiles_permute_kernel(const int4* __restrict__ src,
                                                            const int32_t* __restrict__ count,
                                                            uint32_t seed, int max_tiles,
                                                            int4* __restrict__ dst) {
  const int n = *count;
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n || i >= max_tiles) return;
  auto gcd = [](unsigned x, unsigned y) {
    while (y) {
      const unsigned r = x % y;
      x = y;
      y = r;
    }
    return x;
  };
  unsigned a = (unsigned)(((unsigned long long)seed * 2654435761ull) % (unsigned)n);
  if (a == 0) a = 1;
  while (gcd(a, (unsigned)n) != 1u) a = a + 1 == (unsigned)n ? 1u : a + 1;
  const unsigned c = (unsigned)(((unsigned long long)seed * 40503ull + 7ull) % (unsigned)n);
  dst[i] = src[((unsigned long long)a * (unsigned)i + c) % (unsigned)n];
}

hipError_t launch_tiles(const int32_t* list_offsets, int nlists, int tile_m, int max_tiles,
                        int32_t* tile_offsets, int4* tiles, uint32_t perm_seed,
                        int4* tiles_tmp, hipStream_t st) {
  hipLaunchKernelGGL(tiles_scan_kernel, dim3(1), dim3(kThreads), 0, st, list_offsets, nlists,
                     tile_m, tile_offsets);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nlists == 0) return e;
  int4* first = perm_seed ? tiles_tmp : tiles;
  hipLaunchKernelGGL(index_tiles_kernel, dim3(nlists), dim3(64), 0, st, list_offsets,
                     tile_offsets, tile_m, first);
  if ((e = hipGetLastError()) != hipSuccess || !perm_seed || max_tiles <= 0) return e;
  hipLaunchKernelGGL(tiles_permute_kernel, dim3((max_tiles + 255) / 256), dim3(256), 0, st,
                     tiles_tmp, tile_offsets + nlists, perm_seed, max_tiles, tiles);
  return hipGetLastError();
}

hipError_t launch_index(const Shape& s, const int32_t* idx, int g0, int ng, int tile_m,
                        int32_t* chunk_counts, int32_t* list_count,
                        int32_t* list_offsets, int32_t* tile_offsets, int4* tiles,
                        uint32_t* entries, long long cap, hipStream_t st) {
  const int nb = s.nb();
  const int nchunks = index_chunks(s);
  const int nranges = (nb + kRange - 1) / kRange;
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
  const int nr = nb < kRange ? nb : kRange;
  const dim3 sgrid(nchunks * nranges, ng, s.b);
  // Staging pays where many slot passes would each put single entries into most runs:
  // at least 8 history slots and fewer than 32 entries per list and chunk on average
  // (64K tokens with 128-key blocks: 0.54 -> 0.40 ms; 1M with 4096-key blocks:
  // 4.03 -> 3.88 ms).  With long runs (128K with 4096-key blocks, 88 entries per list
  // and chunk) or few slots (32K, two), the direct writes are already whole lines and
  // the staging only adds its scan (0.28 -> 0.31 ms and 0.04 -> 0.05 ms).
  const long long per_chunk = (long long)kChunk * (s.topk - 1);
  const bool staged = nr <= kStageMaxRange && per_chunk <= kStageEntries &&
                      s.topk - 1 >= 8 && per_chunk < 32ll * nb;
  if (staged) {
    hipLaunchKernelGGL(index_scatter_kernel<true>, sgrid, dim3(kThreads),
                       7 * nr * sizeof(int32_t) + kStageEntries * (sizeof(uint32_t) + sizeof(uint16_t)),
                       st, idx, s.seqs(), s.hq, s.G(), s.block, s.topk, nb, g0, ng, nchunks,
                       chunk_counts, list_count, list_offsets, entries, cap);
  } else {
    hipLaunchKernelGGL(index_scatter_kernel<false>, sgrid, dim3(kThreads),
                       6 * nr * sizeof(int32_t), st, idx, s.seqs(), s.hq, s.G(), s.block,
                       s.topk, nb, g0, ng, nchunks, chunk_counts, list_count, list_offsets,
                       entries, cap);
  }
  return hipGetLastError();
}

}  // namespace moba
