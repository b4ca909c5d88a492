// Backward of the block-sparse attention: dQ, dK, dV for the training use of MoBA
// ("MoBA: Mixture of Block Attention for Long-Context LLMs", README bullet "Trainable
// Block Sparse Attention").  The block selection of the forward is held fixed: it is a
// top-k over inner products with parameter-less mean keys, piecewise constant, so it
// carries no gradient.  Each row is softmax attention over its attended keys N:
//   p_u = exp(scale q.k_u - lse),  dp_u = dO.v_u,  dz_u = p_u (dp_u - D),  D = dO.out,
//   dq = scale sum_u dz_u k_u,  dk_u += scale dz_u q,  dv_u += p_u dO.
// lse and out come from the forward, so p is recomputed without a running max.
//
// Kernels:
//   bwd_delta_kernel   D = rowsum(dO * out) per (b, h, t)
//   bwd_dq_kernel      per row tile, over the keys of one block: S^T = K Q^T,
//                      dP^T = V dO^T, dS^T = P^T (dP^T - D), dQ^T += K^T dS^T.  History
//                      tiles (the inverted index's gathered rows) write an fp32 partial
//                      per (row, slot); current-block tiles add the row's partials to
//                      their own and write dq.
//   bwd_densify_kernel the Q and dO rows (and lse, D) of every index entry, copied
//                      into entry order so that the dK/dV kernel reads them contiguously
//   bwd_dkdv_kernel    per 128 keys of one block: every row that attends them (the
//                      block's history list, then the block's own rows causally) in
//                      groups of 64: S = Q K^T, dP = dO V^T, P, dS, then
//                      dV^T += dO^T P and dK^T += Q^T dS; dK and dV stay in registers
//                      and each key is written by exactly one workgroup.
// MFMA layouts are those of the forward (v_mfma_f32_32x32x16_bf16): a 32x32 result
// lane l holds column l%32 and rows (i/4)*8 + (l/32)*4 + i%4, and a transposed operand
// is read from a row-major LDS tile with ds_read_b64_tr_b16 in the order the result
// registers hold the summation index.  Tiles read both ways are stored once, with their
// 16-byte chunks permuted per row (kv_swz below).

#include "moba_internal.h"

namespace moba {
namespace {

constexpr int kBwdWaves = 8;                // dQ kernel
constexpr int kBwdThreads = 64 * kBwdWaves;
constexpr int kKvTiles = 4;                 // dK/dV kernel: 32-key tiles per workgroup,
constexpr int kKvThreads = 2 * 64 * kKvTiles;   // two waves each
#ifndef MOBA_BWD_KN
#define MOBA_BWD_KN 128
#endif
constexpr int kBwdKN = MOBA_BWD_KN;         // keys per subtile in the dQ kernel (64, 128)
constexpr float kLog2e = 1.4426950408889634f;

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

// ds_read_b64_tr_b16: within each group of 16 lanes, lane i receives element i%4 of
// the 8 bytes addressed by lanes 4j + i/4, j = 0..3.
__device__ __forceinline__ u32x2_t tr16(const char* p) {
  const s16x4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(p));
  return __builtin_bit_cast(u32x2_t, r);
}

// 16 bytes of global memory through a buffer descriptor covering `bytes` from base
// (reads past the end return zero)
__device__ __forceinline__ u32x4_t load16(const void* base, int bytes, int off) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// the B operand of one row (k-step s: dims 16s + 8hf .. +7), zero when !valid
template <int D>
__device__ __forceinline__ void load_row_operand(bf16x8_t (&x)[D / 16], const uint16_t* row,
                                                 bool valid) {
  const int hf = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (valid) v = *reinterpret_cast<const u32x4_t*>(row + 16 * s + 8 * hf);
    x[s] = as_bf16x8(v);
  }
}

}  // namespace

// ------------------------------------------------------------------- D = rowsum(dO*O)
// rows are (token, head) of the [tokens, hq, d] tensors; delta is laid out like lse.
// d/8 consecutive lanes share a row, one 16-byte chunk of out and of dout each, so the
// loads of a wavefront cover whole rows; the lanes' sums are then added pairwise.
__global__ __launch_bounds__(256) void bwd_delta_kernel(const uint16_t* __restrict__ out,
                                                        const uint16_t* __restrict__ dout,
                                                        SeqMap sq, int hq, int d, long rows,
                                                        float* __restrict__ delta) {
  const int lsh = d == 128 ? 4 : 3;                       // lanes per row: 16 or 8
  const long r = ((long)blockIdx.x * 256 + threadIdx.x) >> lsh;  // row token*hq + h
  const int lpr = 1 << lsh, c = (int)(threadIdx.x & (lpr - 1)) * 8;
  float acc = 0.f;
  if (r < rows) {
    const u32x4_t a = *reinterpret_cast<const u32x4_t*>(out + r * d + c);
    const u32x4_t b = *reinterpret_cast<const u32x4_t*>(dout + r * d + c);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      acc += bf16lo(a[e]) * bf16lo(b[e]) + bf16hi(a[e]) * bf16hi(b[e]);
  }
  // every lane takes part in the exchanges (rows past the end add zeros)
  for (int o = lpr / 2; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
  if (r >= rows || c != 0) return;
  const long h = r % hq, token = r / hq;
  if (sq.cu) delta[h * sq.total + token] = acc;
  else delta[((token / sq.T) * hq + h) * sq.T + token % sq.T] = acc;
}

// Row tiles that are read both as MFMA operand rows and with the transpose read (the
// dQ kernel's K subtiles, the dK/dV kernel's Q and dO row groups; V in the dQ kernel
// too) are stored once, unpadded (2D bytes per row), with the 16-byte chunks of row r
// permuted: chunk c sits at position c ^ kv_swz<D>(r).  That one copy serves both
// reads without bank conflicts: the operand read (16 rows, one chunk each, per LDS
// pass) needs the 16 rows' chunks on distinct 16-byte bank groups, and the transpose
// read (4 rows x 64 bytes per pass, rows 4i .. 4i+3) needs the four rows' 64-byte
// spans on distinct quarters of the 256-byte bank line.  (Padded rows serve one of the
// two reads each, so they needed two copies.)
//   D = 128 (16 chunks a row, one row a line): bits 0-1 of r pick the 64-byte quarter,
//           bits 2-3 the chunk within it;
//   D = 64 (8 chunks a row, two rows a line): with x = bits 1-3 of r, bit 0 of x picks
//           the 64-byte half of the row and bits 1-2 the chunk within it.
// kv_swz depends on r mod 16 only, so every 16-row step keeps the permutation.
template <int D>
__device__ __forceinline__ int kv_swz(int r) {
  if constexpr (D == 128) {
    return ((r & 3) << 2) | ((r >> 2) & 3);
  } else {
    const int x = (r >> 1) & 7;
    return ((x & 1) << 2) | (x >> 1);
  }
}

// byte offset of byte `col` (< 2D) of row r in a swizzled group tile
template <int D>
__device__ __forceinline__ int kv_off(int r, int col) {
  return r * (2 * D) + (((col >> 4) ^ kv_swz<D>(r)) << 4) + (col & 15);
}

// A = X^T for rows 16ks .. 16ks+15 of a swizzled group tile, dims dt*32 .. +31, in the
// order the result registers hold the summation index
template <int D>
__device__ __forceinline__ bf16x8_t read_t_swz(const char* tile, int ks, int dt) {
  const int lane = threadIdx.x & 63, hf = lane >> 5;
  const int r = 4 * hf + ((lane & 15) >> 2);            // < 8: rows r and r + 8
  const int col = 32 * ((lane >> 4) & 1) + 8 * (lane & 3) + dt * 64;
  const char* p = tile + 16 * ks * (2 * D);             // kv_swz(16 ks + r) = kv_swz(r)
  const u32x2_t lo = tr16(p + kv_off<D>(r, col));
  const u32x2_t hi = tr16(p + kv_off<D>(r + 8, col));
  return as_bf16x8(u32x4_t{lo[0], lo[1], hi[0], hi[1]});
}

// ------------------------------------------------------------------------- dQ kernel
// One workgroup = kBwdWaves * 32 rows against the keys [kbeg, kend) of one kv-head.
// History: a tile of the inverted index (rows that chose block j; no mask), writing
// the rows' fp32 partials.  Current: 32-token sub-tiles of block c for the query heads
// of kv-head g (as the forward), causal, then the sum with the history partials.
template <int D>
struct DqLds {
  static constexpr int KR = kBwdKN * 2 * D;   // K rows (swizzled): S^T = K Q^T and K^T
  static constexpr int VR = kBwdKN * 2 * D;   // V rows (swizzled) for dP^T = V dO^T
  static constexpr int BUF = KR + VR;
  static constexpr int TOTAL = 2 * BUF;
};

template <int D, bool CUR>
__global__ __launch_bounds__(kBwdThreads, 2) void bwd_dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
    const float* __restrict__ lse, const float* __restrict__ delta, SeqMap sq, int hq,
    int hkv, int block, int topk, float sl, float scale, int g0, int ng, int nb,
    const int4* __restrict__ tiles, const int32_t* __restrict__ tile_count,
    const uint32_t* __restrict__ entries, float* __restrict__ dq_part,
    uint16_t* __restrict__ dq) {
  using L = DqLds<D>;
  constexpr int KS = D / 16, CPR = D / 8;
  __shared__ __attribute__((aligned(16))) char lds[L::TOTAL];
  const int G = hq / hkv, KH = topk - 1;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, n = lane & 31, hf = lane >> 5;
  int b, gi, kbeg, kend, t, hl, slot = 0;
  bool valid;
  if (!CUR) {
    const int tile_id = blockIdx.x;
    if (tile_id >= *tile_count) return;
    const int4 tl = tiles[tile_id];
    const int list = tl.x;
    const int j = list % nb;
    gi = (list / nb) % ng;
    b = list / (nb * ng);
    kbeg = j * block;
    kend = kbeg + block;
    const int e = tl.y + wave * 32 + n;
    valid = e < tl.z;
    const uint32_t ent = valid ? entries[e] : 0u;
    const int sb = entry_slot_bits(topk);
    slot = (int)(ent & ((1u << sb) - 1u));
    t = (int)(ent >> sb) / G;
    hl = (int)(ent >> sb) % G;
  } else {
    // blockIdx.x: a 32*TS-token tile of block blockIdx.y (from the end of the block,
    // longest first) for the GA heads hg*GA .. of kv-head group gi; wave w takes head
    // w % GA and token sub-tile w / GA.  Waves past GA*TS (G not dividing the wave
    // count) and heads past G run on zero rows, so every wave reaches every barrier.
    // Workgroup L (x fastest) runs on XCD L % 8; when the (block, head group) lists
    // number a multiple of 8, each XCD takes whole lists, so the workgroups that stage
    // one block's K/V share one L2 (as the forward's current-block kernel does).
    int bx = blockIdx.x, by = blockIdx.y, bz = blockIdx.z;
    if ((gridDim.y * gridDim.z) % 8 == 0) {
      const int L = bx + gridDim.x * (by + gridDim.y * bz);
      const int xcd = L % 8, i = L / 8;
      const int list = xcd + 8 * (i / gridDim.x);
      bx = i % gridDim.x;
      by = list % gridDim.y;
      bz = list / gridDim.y;
    }
    const int c = by;
    const int GA = G < kBwdWaves ? G : kBwdWaves;   // heads per workgroup
    const int HG = (G + GA - 1) / GA;               // head groups per kv-head
    const int TS = kBwdWaves / GA;                  // 32-token sub-tiles per workgroup
    const int TT = 32 * TS;
    const int hg = bz % HG;
    gi = (bz / HG) % ng;
    b = bz / (HG * ng);
    const int x = gridDim.x - 1 - bx;
    const int t0 = c * block + x * TT;
    const bool active = wave < GA * TS && hg * GA + wave % GA < G;
    hl = active ? hg * GA + wave % GA : 0;
    t = t0 + (wave / GA) * 32 + n;
    kbeg = c * block;
    // a partial last block, or a block past the end of a shorter packed sequence
    kend = min(min(t0 + TT, (c + 1) * block), sq.len(b));
    if (t0 >= kend) return;
    valid = active && t < kend;
    if (!valid) t = c * block;
  }
  const int g = g0 + gi, h = g * G + hl;
  const int tok0 = sq.tok0(b);
  const size_t rs = (size_t)hkv * D;
  const uint16_t* kbase = k + ((size_t)tok0 * hkv + g) * D;
  const uint16_t* vbase = v + ((size_t)tok0 * hkv + g) * D;
  // the row's operands and statistics
  bf16x8_t bq[KS], bo[KS];
  const size_t qrow = ((size_t)tok0 + t) * hq + h;
  load_row_operand<D>(bq, q + qrow * D, valid);
  load_row_operand<D>(bo, dout + qrow * D, valid);
  const size_t lrow = sq.lrow(b, h, hq) + t;
  const float lse2 = valid ? lse[lrow] * kLog2e : 0.f;
  const float dlt = valid ? delta[lrow] : 0.f;
  f32x16_t acc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[dt][i] = 0.f;

  // staging: every thread moves NC 16-byte chunks of the K subtile and of the V subtile
  constexpr int NC = (kBwdKN * CPR + kBwdThreads - 1) / kBwdThreads;
  u32x4_t rk[NC], rv[NC];
  const int nsub = (kend - kbeg + kBwdKN - 1) / kBwdKN;
  auto load_sub = [&](int i) {
    const int kb = kbeg + i * kBwdKN;
    const int nvalid = min(kBwdKN, kend - kb);
    const int bytes = (int)(nvalid * rs * sizeof(uint16_t));
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int ci = min((int)threadIdx.x + c * kBwdThreads, kBwdKN * CPR - 1);
      const int off = (int)(((ci / CPR) * rs + (ci % CPR) * 8) * sizeof(uint16_t));
      rk[c] = load16(kbase + (size_t)kb * rs, bytes, off);
      rv[c] = load16(vbase + (size_t)kb * rs, bytes, off);
    }
  };
  auto store_sub = [&](int buf) {
    char* base = lds + buf * L::BUF;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int ci = threadIdx.x + c * kBwdThreads;
      if ((kBwdKN * CPR) % kBwdThreads == 0 || ci < kBwdKN * CPR) {
        const int row = ci / CPR, col = (ci % CPR) * 16;
        *reinterpret_cast<u32x4_t*>(base + kv_off<D>(row, col)) = rk[c];
        *reinterpret_cast<u32x4_t*>(base + L::KR + kv_off<D>(row, col)) = rv[c];
      }
    }
  };
  load_sub(0);
  store_sub(0);
  __syncthreads();
  for (int i = 0; i < nsub; ++i) {
    if (i + 1 < nsub) load_sub(i + 1);
    const char* kr = lds + (i & 1) * L::BUF;
    const char* vr = kr + L::KR;
    const int kb = kbeg + i * kBwdKN;
    // per 32-key half kk: S^T and dP^T (16 MFMAs), then P^T and dS^T (keys past kend,
    // and in the current block keys after t, get p = 0), then dQ^T += K^T dS^T over the
    // half's two k-steps.  Only one half's scores are live at a time (233 VGPRs instead
    // of 252 for the whole subtile at once; the sums run in the same order).
    const int sw = kv_swz<D>(n);
    auto scores = [&](int kk, f32x16_t& sk, f32x16_t& pk) {
#pragma unroll
      for (int e = 0; e < 16; ++e) sk[e] = pk[e] = 0.f;
      const char* kp = kr + (kk * 32 + n) * (2 * D);
      const char* vp = vr + (kk * 32 + n) * (2 * D);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int co = ((2 * ks + hf) ^ sw) << 4;
        sk = mfma32x32x16(as_bf16x8(*reinterpret_cast<const u32x4_t*>(kp + co)), bq[ks], sk);
        pk = mfma32x32x16(as_bf16x8(*reinterpret_cast<const u32x4_t*>(vp + co)), bo[ks], pk);
      }
    };
    auto dsop = [&](int kk, const f32x16_t& sk, const f32x16_t& pk, bf16x8_t (&d2)[2]) {
      float x[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int u = kb + kk * 32 + (e >> 2) * 8 + hf * 4 + (e & 3);
        const bool keep = u < kend && (!CUR || u <= t);
        const float p = keep ? __builtin_amdgcn_exp2f(fmaf(sk[e], sl, -lse2)) : 0.f;
        x[e] = p * (pk[e] - dlt);
      }
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(x[8 * hh + 2 * e], x[8 * hh + 2 * e + 1]);
        d2[hh] = as_bf16x8(u32x4_t{w[0], w[1], w[2], w[3]});
      }
    };
    auto dqh = [&](int kk, const bf16x8_t (&d2)[2]) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
          acc[dt] = mfma32x32x16(read_t_swz<D>(kr, 2 * kk + hh, dt), d2[hh], acc[dt]);
    };
#pragma unroll
    for (int kk = 0; kk < kBwdKN / 32; ++kk) {
      f32x16_t sk, pk;
      bf16x8_t d2[2];
      scores(kk, sk, pk);
      // the exponentials at raised priority, next to the other wave's MFMAs
      __builtin_amdgcn_s_setprio(1);
      dsop(kk, sk, pk, d2);
      __builtin_amdgcn_s_setprio(0);
      dqh(kk, d2);
    }
    if (i + 1 < nsub) store_sub((i + 1) & 1);
    __syncthreads();
  }

  if (!valid) return;
  const int ngq = ng * G;
  const size_t prow = (sq.prow(b, gi * G + hl, ngq) + t) * KH;
  if (!CUR) {
    float* po = dq_part + (prow + slot) * D + hf * 4;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        f32x4_t w;
#pragma unroll
        for (int r = 0; r < 4; ++r) w[r] = acc[dt][ii * 4 + r] * scale;
        *reinterpret_cast<f32x4_t*>(po + dt * 32 + ii * 8) = w;
      }
    return;
  }
  // current block: this part plus the row's history partials
  const int nh = min(t / block, KH);
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[dt][e] *= scale;
  for (int sidx = 0; sidx < nh; ++sidx) {
    const float* pp = dq_part + (prow + sidx) * D + hf * 4;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const f32x4_t w = *reinterpret_cast<const f32x4_t*>(pp + dt * 32 + ii * 8);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[dt][ii * 4 + r] += w[r];
      }
  }
  uint16_t* orow = dq + qrow * D + hf * 4;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      u32x2_t pk;
      pk[0] = f32_to_bf16_rne(acc[dt][ii * 4]) | (f32_to_bf16_rne(acc[dt][ii * 4 + 1]) << 16);
      pk[1] = f32_to_bf16_rne(acc[dt][ii * 4 + 2]) | (f32_to_bf16_rne(acc[dt][ii * 4 + 3]) << 16);
      *reinterpret_cast<u32x2_t*>(orow + dt * 32 + ii * 8) = pk;
    }
}

// ------------------------------------------------------------------------ densify
// Copies, for every entry e of the inverted index (one workgroup per index tile of up
// to 256 entries of one list (b, g, j)), the entry's Q row and dO row to rows[e] =
// [q | dout] (2 D bf16) and its lse and delta to meta[e] = [lse, delta]: the history
// rows of each block in list order, contiguous, for the dK/dV kernel.
template <int D>
__global__ __launch_bounds__(256) void bwd_densify_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ dout,
    const float* __restrict__ lse, const float* __restrict__ delta, SeqMap sq, int hq, int G,
    int g0, int ng, int nb, int sbits, const int4* __restrict__ tiles,
    const int32_t* __restrict__ tile_count, const uint32_t* __restrict__ entries,
    uint16_t* __restrict__ rows, float* __restrict__ meta) {
  constexpr int CPR = D / 8;
  if ((int)blockIdx.x >= *tile_count) return;
  const int4 tl = tiles[blockIdx.x];
  const int list = tl.x, e0 = tl.y, ne = tl.z - tl.y;
  const int gi = (list / nb) % ng, b = list / (nb * ng);
  const int hb = (g0 + gi) * G, tok0 = sq.tok0(b);
  for (int x = threadIdx.x; x < ne * 2 * CPR; x += 256) {
    const int e = e0 + x / (2 * CPR), which = (x / CPR) & 1, col = (x % CPR) * 8;
    const uint32_t rr = entries[e] >> sbits;
    const int t = (int)rr / G, h = hb + (int)rr % G;
    const uint16_t* src = (which ? dout : q) + (((size_t)tok0 + t) * hq + h) * D + col;
    *reinterpret_cast<u32x4_t*>(rows + ((size_t)e * 2 + which) * D + col) =
        *reinterpret_cast<const u32x4_t*>(src);
  }
  if ((int)threadIdx.x < ne) {
    const int e = e0 + threadIdx.x;
    const uint32_t rr = entries[e] >> sbits;
    const int t = (int)rr / G, h = hb + (int)rr % G;
    const size_t at = sq.lrow(b, h, hq) + t;
    meta[(size_t)e * 2] = lse[at];
    meta[(size_t)e * 2 + 1] = delta[at];
  }
}

// ----------------------------------------------------------------------- dK/dV kernel
// One workgroup = 32 * kKvTiles keys of block j of kv-head g.  Rows: the history list
// of (b, g, j) from the inverted index, then the rows of block j from token kc0 on
// (causal: key u is attended by token t >= u), G heads each, in groups of kKvRG.
// Each 32-key tile has two waves on one SIMD: wave "P" computes S = Q K^T, P, and
// dV^T += dO^T P; wave "dS" computes dP = dO V^T, takes P through LDS, and
// dK^T += Q^T dS with dS = P (dP - D).  Each wave keeps one 32 x D accumulator and one
// B operand, so two waves fit per SIMD and one's VALU work overlaps the other's MFMAs.
// The history rows are read from bwd_densify_kernel's copy: every workgroup of the
// block streams the same contiguous rows instead of gathering them from all over Q.
#ifndef MOBA_KV_RG
#define MOBA_KV_RG 64
#endif
constexpr int kKvRG = MOBA_KV_RG;     // rows per staged group: 32 or 64
constexpr int kKvRB = kKvRG / 32;     // 32-row MFMA blocks per group
static_assert(kKvRG == 32 || kKvRG == 64, "groups of one or two 32-row blocks");

template <int D>
struct KvLds {
  static constexpr int RB = 2 * D;                      // bytes per row
  static constexpr int QB = kKvRG * RB;                 // Q (or dO) rows of a group
  static constexpr int BUF = 2 * QB + 3 * kKvRG * 4;    // Q, dO; lse2, delta, t
  static constexpr int PX = kKvTiles * kKvRB * 64 * 32; // P, 32 bytes per lane and block
  static constexpr int TOTAL = 2 * BUF + PX;
};

// HFAST: groups made only of history rows load them from one scalar base with fixed
// per-thread offsets.  Chosen for long blocks, whose lists are long (128K with
// B = 4096: 0.4% faster); with B = 512 at 32K the general path alone was faster.
template <int D, bool POW2, bool HFAST>
__global__ __launch_bounds__(kKvThreads, 2) void bwd_dkdv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
    const float* __restrict__ lse, const float* __restrict__ delta, SeqMap sq, int hq,
    int hkv, int block, float sl, float scale, int g0, int ng, int nb,
    const int32_t* __restrict__ list_offsets, const uint16_t* __restrict__ dense_rows,
    const float* __restrict__ dense_meta, uint16_t* __restrict__ dk,
    uint16_t* __restrict__ dv) {
  using L = KvLds<D>;
  constexpr int KS = D / 16, CPR = D / 8;
  __shared__ __attribute__((aligned(16))) char lds[L::TOTAL];
  const int G = hq / hkv;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, n = lane & 31, hf = lane >> 5;
  const int tile = wave % kKvTiles;
  const bool role_ds = wave >= kKvTiles;      // false: S, P, dV   true: dP, dS, dK
  // work item: key chunk fastest, then block, then (b, kv-head)
  const int W = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
  const int wx = W % gridDim.x, wyz = W / gridDim.x;
  const int j = wyz % gridDim.y, gi = (wyz / gridDim.y) % ng, b = wyz / (gridDim.y * ng);
  const int g = g0 + gi;
  const int kc0 = j * block + wx * 32 * kKvTiles;
  const int u = kc0 + tile * 32 + n;                  // this lane's key
  // a partial last block, or a block past the end of a shorter packed sequence
  const int kend = min((j + 1) * block, sq.len(b));
  if (kc0 >= kend) return;
  const int tok0 = sq.tok0(b);
  const bool kvalid = u < kend;
  const int list = (b * ng + gi) * nb + j;
  const int hbeg = list_offsets ? list_offsets[list] : 0;
  const int nhist = list_offsets ? list_offsets[list + 1] - hbeg : 0;
  // tokens of block j before kc0 attend none of these keys
  const int nrows = nhist + (kend - kc0) * G;
  // the K (wave P) or V (wave dS) row of this lane's key: the B operand, lane = key
  bf16x8_t bkv[KS];
  load_row_operand<D>(bkv,
                      (role_ds ? v : k) + (((size_t)tok0 + (kvalid ? u : kc0)) * hkv + g) * D,
                      kvalid);
  f32x16_t acc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[dt][i] = 0.f;

  // Staging of a group: thread x moves 16-byte chunk x % (kKvRG*CPR) of Q (x <
  // kKvRG*CPR) or of dO; threads 0..kKvRG-1 also the rows' lse2, delta and causal
  // limit t.  History rows come from the densified copy of the list (entry order,
  // contiguous); the block's own rows are token kc0 + rc / G, head rc % G.  Rows past
  // the end read a valid row and get p = 0 from lse2 = +inf, so the fetch has no
  // branches.  Group i+1 is in flight while group i is computed.
  constexpr int CHUNKS = 2 * kKvRG * CPR;
  constexpr int NC = CHUNKS / kKvThreads;
  static_assert(CHUNKS % kKvThreads == 0, "every thread moves whole chunks");
  // own-block row rc is token kc0 + rc / G, head rc % G (shifts when G is a power of 2)
  const int gshift = __builtin_ctz((unsigned)G);
  auto rtok = [&](int rc) {
    if constexpr (POW2) return rc >> gshift;
    else return rc / G;
  };
  auto rhead = [&](int rc) {
    if constexpr (POW2) return rc & (G - 1);
    else return rc % G;
  };
  const size_t row_base = (size_t)tok0 * hq + g * G;   // row of (b, t = 0, head g*G)
  const size_t meta_base = sq.lrow(b, g * G, hq);     // lse/delta of (b, g*G, t = 0)
  const int lhs = sq.lhead();                          // lse stride between heads
  int crow[NC], ccol[NC], soff[NC];
  bool cdo[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int x = threadIdx.x + c * kKvThreads;
    cdo[c] = x >= kKvRG * CPR;
    crow[c] = (x % (kKvRG * CPR)) / CPR;
    ccol[c] = (x % CPR) * 8;
    soff[c] = (cdo[c] ? L::QB : 0) + kv_off<D>(crow[c], ccol[c] * 2);
  }
  struct Rows {
    u32x4_t c[NC];
    float f, d;
    int t;
  };
  // the q (dO) row of current row r >= nhist (clamped to the last row past the end)
  auto cur_row = [&](int r) -> size_t {
    const int rc = min(r, nrows - 1) - nhist;
    return row_base + (size_t)(kc0 + rtok(rc)) * hq + rhead(rc);
  };
  // element offset of this thread's chunks within a group of densified history rows
  int hoff[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) hoff[c] = (crow[c] * 2 + cdo[c]) * D + ccol[c];
  auto fetch_rows = [&](int r0, Rows& rd) {
    if constexpr (HFAST) {
      if (r0 + kKvRG <= nhist) {
        const uint16_t* hb = dense_rows + (size_t)(hbeg + r0) * 2 * D;
#pragma unroll
        for (int c = 0; c < NC; ++c)
          rd.c[c] = *reinterpret_cast<const u32x4_t*>(hb + hoff[c]);
        const float* m = dense_meta + (size_t)(hbeg + r0 + (threadIdx.x & (kKvRG - 1))) * 2;
        rd.f = m[0] * kLog2e;
        rd.d = m[1];
        rd.t = 0x7fffffff;
        return;
      }
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int r = r0 + crow[c];
      const uint16_t* hsrc = dense_rows + ((size_t)(hbeg + r) * 2 + cdo[c]) * D;
      const uint16_t* csrc = (cdo[c] ? dout : q) + cur_row(r) * D;
      rd.c[c] = *reinterpret_cast<const u32x4_t*>((r < nhist ? hsrc : csrc) + ccol[c]);
    }
    const int r = r0 + (threadIdx.x & (kKvRG - 1));
    float lv, dv0;
    if (r < nhist) {
      const float* m = dense_meta + (size_t)(hbeg + r) * 2;
      lv = m[0];
      dv0 = m[1];
    } else {
      const int rc = min(r, nrows - 1) - nhist;
      const size_t at = meta_base + (size_t)rhead(rc) * lhs + kc0 + rtok(rc);
      lv = lse[at];
      dv0 = delta[at];
    }
    rd.f = r < nrows ? lv * kLog2e : INFINITY;   // p = 0 for rows past the end
    rd.d = r < nrows ? dv0 : 0.f;
    rd.t = r < nhist ? 0x7fffffff : kc0 + rtok(min(r, nrows - 1) - nhist);
  };
  auto store_rows = [&](const Rows& rd, int buf) {
    char* base = lds + buf * L::BUF;
#pragma unroll
    for (int c = 0; c < NC; ++c) *reinterpret_cast<u32x4_t*>(base + soff[c]) = rd.c[c];
    if (threadIdx.x < kKvRG) {
      float* mf = reinterpret_cast<float*>(base + 2 * L::QB);
      mf[threadIdx.x] = rd.f;
      mf[kKvRG + threadIdx.x] = rd.d;
      reinterpret_cast<int*>(mf + 2 * kKvRG)[threadIdx.x] = rd.t;
    }
  };
  // rows nhist + (0 .. 32*kKvTiles*G - 1) are the tokens kc0 .. kc0 + 32*kKvTiles - 1,
  // the only ones that see keys after themselves; other groups need no causal mask
  const int mask_lo = nhist, mask_hi = nhist + 32 * kKvTiles * G;
  // this lane's P slots: per 32-row block two 16-byte planes 1 KB apart, so that the
  // 64 lanes of a 16-byte access touch consecutive bytes
  char* px = lds + 2 * L::BUF + tile * (kKvRB * 2048) + lane * 16;
  // this lane's operand-row offset (row n of each 32-row block, k-step 0)
  const int aoff = n * (2 * D);
  const int aswz = kv_swz<D>(n);
  // One group.  Register e of a 32x32 result holds row (e/4)*8 + hf*4 + e%4 of its
  // 32-row block.  One code path for both buffers and with or without the causal mask
  // (a uniform branch around the mask alone): copies of it for each case had the
  // compiler keep the accumulators in different registers in each copy and move them
  // between them.
  auto compute = [&](int buf, bool masked) {
    const char* base = lds + buf * L::BUF;
    const float* mf = reinterpret_cast<const float*>(base + 2 * L::QB);
    // S = Q K^T (wave P) or dP = dO V^T (wave dS): rows x keys, one chain per 32-row
    // block, the chains alternating
    const char* ar = base + (role_ds ? L::QB : 0) + aoff;
    f32x16_t sc[kKvRB];
#pragma unroll
    for (int rb = 0; rb < kKvRB; ++rb) sc[rb] = f32x16_t{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int rb = 0; rb < kKvRB; ++rb)
        sc[rb] = mfma32x32x16(
            as_bf16x8(*reinterpret_cast<const u32x4_t*>(
                ar + rb * 32 * (2 * D) + (((2 * ks + hf) ^ aswz) << 4))),
            bkv[ks], sc[rb]);
    bf16x8_t op[2 * kKvRB];
    if (!role_ds) {
#pragma unroll
      for (int rb = 0; rb < kKvRB; ++rb) {
        float p[16];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x4_t lf =
              *reinterpret_cast<const f32x4_t*>(mf + rb * 32 + q4 * 8 + hf * 4);
#pragma unroll
          for (int r = 0; r < 4; ++r)
            p[q4 * 4 + r] = __builtin_amdgcn_exp2f(fmaf(sc[rb][q4 * 4 + r], sl, -lf[r]));
        }
        if (masked) {
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const int4 lt = *reinterpret_cast<const int4*>(mf + 2 * kKvRG + rb * 32 +
                                                           q4 * 8 + hf * 4);
            const int tt[4] = {lt.x, lt.y, lt.z, lt.w};
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (u > tt[r]) p[q4 * 4 + r] = 0.f;
          }
        }
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          uint32_t w[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            w[e] = pack_bf16x2(p[8 * hh + 2 * e], p[8 * hh + 2 * e + 1]);
          op[2 * rb + hh] = as_bf16x8(u32x4_t{w[0], w[1], w[2], w[3]});
          *reinterpret_cast<u32x4_t*>(px + 1024 * (2 * rb + hh)) =
              u32x4_t{w[0], w[1], w[2], w[3]};
        }
      }
    }
    __syncthreads();   // P of every tile is in LDS
    // Wave dS runs the second phase at raised priority: its dS VALU and then its dK
    // MFMAs issue first and wave P's dV MFMAs fill the gaps, so the two waves of a SIMD
    // reach the next barrier together instead of wave dS finishing alone.
    if (role_ds) {
      __builtin_amdgcn_s_setprio(1);
      // dS = P (dP - D), P as rounded to bf16 by wave P
#pragma unroll
      for (int rb = 0; rb < kKvRB; ++rb) {
        const u32x4_t pw0 = *reinterpret_cast<const u32x4_t*>(px + 1024 * (2 * rb));
        const u32x4_t pw1 = *reinterpret_cast<const u32x4_t*>(px + 1024 * (2 * rb + 1));
        const uint32_t pw[8] = {pw0[0], pw0[1], pw0[2], pw0[3],
                                pw1[0], pw1[1], pw1[2], pw1[3]};
        float x[16];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x4_t ld =
              *reinterpret_cast<const f32x4_t*>(mf + kKvRG + rb * 32 + q4 * 8 + hf * 4);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int e = q4 * 4 + r;
            const float pe = (e & 1) ? bf16hi(pw[e >> 1]) : bf16lo(pw[e >> 1]);
            x[e] = pe * (sc[rb][e] - ld[r]);
          }
        }
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          uint32_t w[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            w[e] = pack_bf16x2(x[8 * hh + 2 * e], x[8 * hh + 2 * e + 1]);
          op[2 * rb + hh] = as_bf16x8(u32x4_t{w[0], w[1], w[2], w[3]});
        }
      }
    }
    // dV^T += dO^T P (wave P) or dK^T += Q^T dS (wave dS), over the group's rows
    const char* tt = base + (role_ds ? 0 : L::QB);
#pragma unroll
    for (int ks = 0; ks < 2 * kKvRB; ++ks)
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
        acc[dt] = mfma32x32x16(read_t_swz<D>(tt, ks, dt), op[ks], acc[dt]);
    if (role_ds) __builtin_amdgcn_s_setprio(0);
  };
  const int ngroups = (nrows + kKvRG - 1) / kKvRG;
  Rows rd;
  fetch_rows(0, rd);             // group 0
  store_rows(rd, 0);
  __syncthreads();
  // groups [gm0, gm1) hold the rows that need the causal mask
  const int gm0 = mask_lo / kKvRG, gm1 = (mask_hi + kKvRG - 1) / kKvRG;
  for (int gidx = 0; gidx < ngroups; ++gidx) {
    fetch_rows((gidx + 1) * kKvRG, rd);     // group gidx + 1
    compute(gidx & 1, gidx >= gm0 && gidx < gm1);
    store_rows(rd, (gidx + 1) & 1);
    __syncthreads();
  }

  if (!kvalid) return;
  const float os = role_ds ? scale : 1.f;
  uint16_t* orow = (role_ds ? dk : dv) + (((size_t)tok0 + u) * hkv + g) * D + hf * 4;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      u32x2_t w;
      w[0] = f32_to_bf16_rne(acc[dt][ii * 4] * os) |
             (f32_to_bf16_rne(acc[dt][ii * 4 + 1] * os) << 16);
      w[1] = f32_to_bf16_rne(acc[dt][ii * 4 + 2] * os) |
             (f32_to_bf16_rne(acc[dt][ii * 4 + 3] * os) << 16);
      *reinterpret_cast<u32x2_t*>(orow + dt * 32 + ii * 8) = w;
    }
}

// ------------------------------------------------------------------------- launchers
int bwd_tile_rows() { return kBwdWaves * 32; }

// the current-block dQ tiles put the G heads of a kv-head on different waves
bool bwd_supported(const Shape& s) { return s.G() >= 1; }

hipError_t launch_bwd_delta(const Shape& s, const uint16_t* out, const uint16_t* dout,
                            float* delta, hipStream_t st) {
  const long rows = (s.cu ? (long)s.total : (long)s.b * s.T) * s.hq;
  const long threads = rows * (s.d / 8);                   // d/8 lanes per row
  hipLaunchKernelGGL(bwd_delta_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                     st, out, dout, s.seqs(), s.hq, s.d, rows, delta);
  return hipGetLastError();
}

hipError_t launch_bwd_dq_history(const Shape& s, const uint16_t* q, const uint16_t* k,
                                 const uint16_t* v, const uint16_t* dout, const float* lse,
                                 const float* delta, float scale, int g0, int ng,
                                 const int4* tiles, const int32_t* tile_count, int max_tiles,
                                 const uint32_t* entries, float* dq_part, hipStream_t st) {
  if (max_tiles <= 0) return hipSuccess;
  const float sl = scale * kLog2e;
#define MOBA_DQH(DD)                                                                       \
  hipLaunchKernelGGL((bwd_dq_kernel<DD, false>), dim3(max_tiles), dim3(kBwdThreads), 0, st, \
                     q, k, v, dout, lse, delta, s.seqs(), s.hq, s.hkv, s.block, s.topk, sl,   \
                     scale, g0, ng, s.nb(), tiles, tile_count, entries, dq_part, nullptr)
  if (s.d == 128) MOBA_DQH(128);
  else MOBA_DQH(64);
#undef MOBA_DQH
  return hipGetLastError();
}

hipError_t launch_bwd_dq_current(const Shape& s, const uint16_t* q, const uint16_t* k,
                                 const uint16_t* v, const uint16_t* dout, const float* lse,
                                 const float* delta, float scale, int g0, int ng,
                                 const float* dq_part, uint16_t* dq, hipStream_t st) {
  const float sl = scale * kLog2e;
  const int GA = s.G() < kBwdWaves ? s.G() : kBwdWaves;     // heads per workgroup
  const int HG = (s.G() + GA - 1) / GA;                     // head groups per kv-head
  const int TT = 32 * (kBwdWaves / GA);
  dim3 grid((s.block + TT - 1) / TT, s.nb(), s.b * ng * HG);
#define MOBA_DQC(DD)                                                                       \
  hipLaunchKernelGGL((bwd_dq_kernel<DD, true>), grid, dim3(kBwdThreads), 0, st, q, k, v,     \
                     dout, lse, delta, s.seqs(), s.hq, s.hkv, s.block, s.topk, sl, scale, g0, \
                     ng, s.nb(), nullptr, nullptr, nullptr, const_cast<float*>(dq_part), dq)
  if (s.d == 128) MOBA_DQC(128);
  else MOBA_DQC(64);
#undef MOBA_DQC
  return hipGetLastError();
}

hipError_t launch_bwd_densify(const Shape& s, const uint16_t* q, const uint16_t* dout,
                              const float* lse, const float* delta, int g0, int ng,
                              const int4* tiles, const int32_t* tile_count, int max_tiles,
                              const uint32_t* entries, uint16_t* rows, float* meta,
                              hipStream_t st) {
  if (max_tiles <= 0) return hipSuccess;
#define MOBA_DENSE(DD)                                                                     \
  hipLaunchKernelGGL((bwd_densify_kernel<DD>), dim3(max_tiles), dim3(256), 0, st, q, dout,  \
                     lse, delta, s.seqs(), s.hq, s.G(), g0, ng, s.nb(),                     \
                     entry_slot_bits(s.topk), tiles, tile_count, entries, rows, meta)
  if (s.d == 128) MOBA_DENSE(128);
  else MOBA_DENSE(64);
#undef MOBA_DENSE
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv(const Shape& s, const uint16_t* q, const uint16_t* k,
                           const uint16_t* v, const uint16_t* dout, const float* lse,
                           const float* delta, float scale, int g0, int ng,
                           const int32_t* list_offsets, const uint16_t* dense_rows,
                           const float* dense_meta, uint16_t* dk, uint16_t* dv,
                           hipStream_t st) {
  const float sl = scale * kLog2e;
  const int kpw = 32 * kKvTiles;
  dim3 grid((s.block + kpw - 1) / kpw, s.nb(), s.b * ng);
#define MOBA_KV(DD, P2, HF)                                                                \
  hipLaunchKernelGGL((bwd_dkdv_kernel<DD, P2, HF>), grid, dim3(kKvThreads), 0, st, q, k, v,  \
                     dout, lse, delta, s.seqs(), s.hq, s.hkv, s.block, sl, scale, g0, ng,     \
                     s.nb(), list_offsets, dense_rows, dense_meta, dk, dv)
  const bool pow2 = (s.G() & (s.G() - 1)) == 0;
  const bool hfast = s.block >= 1024;
  if (s.d == 128) {
    if (pow2 && hfast) MOBA_KV(128, true, true);
    else if (pow2) MOBA_KV(128, true, false);
    else if (hfast) MOBA_KV(128, false, true);
    else MOBA_KV(128, false, false);
  } else {
    if (pow2 && hfast) MOBA_KV(64, true, true);
    else if (pow2) MOBA_KV(64, true, false);
    else if (hfast) MOBA_KV(64, false, true);
    else MOBA_KV(64, false, false);
  }
#undef MOBA_KV
  return hipGetLastError();
}

}  // namespace moba
