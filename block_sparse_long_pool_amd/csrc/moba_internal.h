// Internal declarations of libmoba: device helpers shared by the kernels and the
// host-side launchers that moba_api.hip strings together.  Written for gfx950
// (CDNA4): 64-lane wavefronts, v_mfma_f32_32x32x16_bf16, 160 KB of LDS per CU.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moba {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kThreads = 256;  // every kernel runs 4 wavefronts per workgroup

// ---------------------------------------------------------------- bf16 helpers
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float -> bf16 bits, round to nearest even (inputs are finite)
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) {
  return __builtin_bit_cast(bf16x8_t, v);
}

// two floats -> packed bf16 pair (v_cvt_pk_bf16_f32 on gfx950)
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2_t r;
  r[0] = (__bf16)a;
  r[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ f32x16_t mfma32x32x16(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// value held by lane (lane ^ 32)
__device__ __forceinline__ uint32_t xor32_u32(uint32_t v) {
  return (uint32_t)__shfl_xor((int)v, 32);
}
__device__ __forceinline__ float xor32_f32(float v) {
  return __uint_as_float(xor32_u32(__float_as_uint(v)));
}

__device__ __forceinline__ int wave_max_i32(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o));
  return v;
}

}  // namespace moba

// ------------------------------------------------------------------ launchers
// Each returns hipSuccess or the launch error.  Shapes were validated by the caller.
namespace moba {

// Token layout.  cu == nullptr: b sequences of T tokens each, tensors [b, T, heads, d],
// lse [b, hq, T], idx [b, hq, T, topk].  Otherwise b packed sequences: sequence i is
// tokens cu[i] .. cu[i+1]-1 of [total, heads, d] tensors, T is at least every length,
// lse is [hq, total] and idx [hq, total, topk].  Each sequence has its own block grid
// starting at its first token; its last block may be partial.
struct SeqMap {
  const int32_t* cu;
  int T, total;
  __device__ __forceinline__ int tok0(int b) const { return cu ? cu[b] : b * T; }
  __device__ __forceinline__ int len(int b) const { return cu ? cu[b + 1] - cu[b] : T; }
  // element index of (b, h, t = 0) in lse; the token stride is 1
  __device__ __forceinline__ size_t lrow(int b, int h, int hq) const {
    return cu ? (size_t)h * total + cu[b] : ((size_t)b * hq + h) * T;
  }
  // stride between the lse rows of two heads of one sequence
  __device__ __forceinline__ int lhead() const { return cu ? total : T; }
  // row of (b, head hh of the ngq heads of a kv-head group, t = 0) in the history
  // partials, [b, ngq, T] or packed [ngq, total]; the token stride is 1
  __device__ __forceinline__ size_t prow(int b, int hh, int ngq) const {
    return cu ? (size_t)hh * total + cu[b] : ((size_t)b * ngq + hh) * T;
  }
};

// Inverted-index entries pack (r << sbits) | slot, r = t*G + h%G the row of a kv-head
// and slot < topk - 1 the position of the block in the row's selection.  Up to 32
// history slots take 5 bits, up to 64 take 6 (rows then have 26 bits).
__host__ __device__ __forceinline__ int entry_slot_bits(int topk) {
  return topk - 1 > 32 ? 6 : 5;
}

struct Shape {
  int b, T, hq, hkv, d, block, topk;
  const int32_t* cu = nullptr;   // packed sequences (device), see SeqMap
  int total = 0;
  int nb() const { return (T + block - 1) / block; }
  int G() const { return hq / hkv; }
  int KH() const { return topk - 1; }
  SeqMap seqs() const { return SeqMap{cu, T, total}; }
};

// (a1) centroid mean-pool
int pool_splits(const Shape& s);
// with chi/clo non-null the same pass also writes the centroids' bf16 hi + lo split
hipError_t launch_pool(const Shape& s, const uint16_t* k, float* partial, float* cent,
                       uint16_t* chi, uint16_t* clo, hipStream_t st);
// fp32 centroids -> bf16 hi + bf16 lo (c ~= hi + lo to ~2^-17 relative)
hipError_t launch_centroid_split(const Shape& s, const float* cent, uint16_t* chi,
                                 uint16_t* clo, hipStream_t st);
// (a2) gate + top-k
hipError_t launch_gate(const Shape& s, const uint16_t* q, const uint16_t* chi,
                       const uint16_t* clo, int32_t* idx, hipStream_t st);
// every row selects all of its causal blocks (topk >= the number of blocks): blocks
// 0 .. t / block ascending, then -1 up to topk
hipError_t launch_idx_all_blocks(const Shape& s, int32_t* idx, hipStream_t st);
int gate_max_history();                // the most history slots the gate ranks
// (a3) inverted index over kv-heads [g0, g0 + ng); tile_offsets as for launch_tiles
int index_chunks(const Shape& s);
hipError_t launch_index(const Shape& s, const int32_t* idx, int g0, int ng, int tile_m,
                        int32_t* chunk_counts, int32_t* list_count,
                        int32_t* list_offsets, int32_t* tile_offsets,
                        int4* tiles, uint32_t* entries, long long cap,
                        hipStream_t st);
// the tile list of lists given by their offsets (as moba_build_index writes them):
// tile_offsets [nlists + 2] (then the tile count, then a zeroed counter that the
// persistent history kernel takes tiles from) and tiles; with perm_seed != 0 the
// tiles are written in a seeded permuted order (through tiles_tmp, max_tiles long)
hipError_t launch_tiles(const int32_t* list_offsets, int nlists, int tile_m, int max_tiles,
                        int32_t* tile_offsets, int4* tiles, uint32_t perm_seed,
                        int4* tiles_tmp, hipStream_t st);
// (a4) history attention partials, (a5) current block fused with the merge
// tile_count: the tile count, then the zeroed queue counter that launch_index and
// launch_tiles write after it (the persistent kernel takes tiles from it)
hipError_t launch_attn_history(const Shape& s, const uint16_t* q, const uint16_t* k,
                               const uint16_t* v, float scale, int g0, int ng,
                               const int4* tiles, int32_t* tile_count,
                               int max_tiles, const uint32_t* entries, uint16_t* part_o,
                               float* part_lse, hipStream_t st);
// the current-block kernel also merges the history partials and writes out and lse
hipError_t launch_attn_current(const Shape& s, const uint16_t* q, const uint16_t* k,
                               const uint16_t* v, float scale, int g0, int ng,
                               const uint16_t* part_o, const float* part_lse, uint16_t* out,
                               float* lse, hipStream_t st);
int history_tile_rows();                    // rows per tile of the streaming kernel
// rows per tile of the kernel s runs on, for a pass of n_entries index entries
int history_tile_rows(const Shape& s, long long n_entries);

// full-attention decode: n new queries at the last n positions of a Tk-key cache, the
// keys split over many wavefronts (fp32 (o, lse) partials per split), then a merge
struct DecodePlan {
  int nsplit, spt;                     // splits, 32-key subtiles per split
  size_t part_o_bytes, part_lse_bytes;
};
DecodePlan decode_plan(int b, int n, int Tk, int hq, int hkv, int d);
int decode_max_rows();                 // bound on (hq / hkv) * n (query rows per kv-head)
hipError_t launch_decode(int b, int n, int Tk, int hq, int hkv, int d, float scale,
                         const DecodePlan& p, const uint16_t* q, const uint16_t* k,
                         const uint16_t* v, float* part_o, float* part_lse, uint16_t* out,
                         float* lse, hipStream_t st);

// short depthwise causal convolution of the keys within blocks (width <= 8)
int conv_max_width();
hipError_t launch_key_conv(const Shape& s, const uint16_t* k, const float* weight, int width,
                           uint16_t* out, hipStream_t st);

// backward with the selection held fixed: D = rowsum(dO * out), dQ over the history
// tiles (fp32 partials per row and slot) and the current blocks (sum -> dq), and dK/dV
// per 32*4 keys of a block over the rows that attend them
bool bwd_supported(const Shape& s);
int bwd_tile_rows();
hipError_t launch_bwd_delta(const Shape& s, const uint16_t* out, const uint16_t* dout,
                            float* delta, hipStream_t st);
hipError_t launch_bwd_dq_history(const Shape& s, const uint16_t* q, const uint16_t* k,
                                 const uint16_t* v, const uint16_t* dout, const float* lse,
                                 const float* delta, float scale, int g0, int ng,
                                 const int4* tiles, const int32_t* tile_count, int max_tiles,
                                 const uint32_t* entries, float* dq_part, hipStream_t st);
hipError_t launch_bwd_dq_current(const Shape& s, const uint16_t* q, const uint16_t* k,
                                 const uint16_t* v, const uint16_t* dout, const float* lse,
                                 const float* delta, float scale, int g0, int ng,
                                 const float* dq_part, uint16_t* dq, hipStream_t st);
// the Q and dO rows and lse/delta of every index entry, in entry order (contiguous)
hipError_t launch_bwd_densify(const Shape& s, const uint16_t* q, const uint16_t* dout,
                              const float* lse, const float* delta, int g0, int ng,
                              const int4* tiles, const int32_t* tile_count, int max_tiles,
                              const uint32_t* entries, uint16_t* rows, float* meta,
                              hipStream_t st);
hipError_t launch_bwd_dkdv(const Shape& s, const uint16_t* q, const uint16_t* k,
                           const uint16_t* v, const uint16_t* dout, const float* lse,
                           const float* delta, float scale, int g0, int ng,
                           const int32_t* list_offsets, const uint16_t* dense_rows,
                           const float* dense_meta, uint16_t* dk, uint16_t* dv,
                           hipStream_t st);

}  // namespace moba
