// Block-sparse attention: history blocks (gather-and-densify) and the causal current
// block, each producing (o, lse) partials, then the log-sum-exp merge.
//
// The method: each query attends the keys of its selected blocks only, the current
// block causally ("MoBA: Mixture of Block Attention for Long-Context LLMs", paper
// summary page, "Approach"; README bullet "Trainable Block Sparse Attention").  The
// history part follows the Gather-and-Densify idea of the FlashMoBA story (hyper.ai):
// the queries that chose one block are gathered into a dense tile and run against
// that block staged on chip.  Splitting a row's keys into parts and merging the
// parts' softmax results by log-sum-exp gives exactly the one-softmax result.
//
// MFMA layout (v_mfma_f32_32x32x16_bf16, one wavefront per 32*QT query rows):
//   scores   S^T[key][query] = K Q^T: A = K rows from LDS, B = Q rows in registers.
//            Lane l holds query l%32 and keys (i/4)*8 + (l/32)*4 + i%4, i < 16, of
//            each 32-key half, so the softmax of a query lives in two lanes
//            (l, l^32) and its running max/sum/scale are per-lane scalars.
//   output   O^T[dim][query] = V^T P^T: B = P^T straight from the score registers
//            (converted to bf16), A = V^T read from the row-major V tile with the
//            gfx950 LDS transpose read (ds_read_b64_tr_b16), whose key order is
//            chosen to match the order the score registers hold the keys in, so no
//            register shuffle and no transpose while staging are needed.
// K and V tiles are row-major in LDS with padded rows (K: +16 B, V: +32 B), which
// spreads the MFMA operand reads over all banks and lets every read use a per-lane
// base address plus an immediate offset.
// Online softmax in the log2 domain (scale * log2(e) folded into one FMA).
#include "moba_internal.h"

namespace moba {

// query rows per wavefront = 32 * QT; waves per SIMD the compiler budgets for
#ifndef MOBA_ATTN_QT
#define MOBA_ATTN_QT 1
#endif
#ifndef MOBA_ATTN_WPE
#define MOBA_ATTN_WPE 2
#endif

constexpr int KN = 64;          // keys per LDS subtile
constexpr float kTau = 8.f;     // lazy rescale: the reference max may lag by 2^8

template <int D>
struct Lds {
  static constexpr int KS = D * 2 + 16;          // K row stride (bytes)
  static constexpr int VS = D * 2 + 32;          // V row stride (bytes)
  static constexpr int KBYTES = KN * KS;
  static constexpr int VBYTES = KN * VS;
  static constexpr int STAGE = KBYTES + VBYTES;  // one K + V subtile
};

template <int D, int QT>
struct WaveState {
  bf16x8_t q[QT][D / 16];
  f32x16_t o[QT][D / 32];
  float m[QT], l[QT];
};

// one subtile of K and V in flight through registers (global -> regs -> LDS)
template <int D>
struct KVRegs {
  static constexpr int CPR = D / 8;                                  // 16 B chunks per row
  static constexpr int NC = (KN * CPR + kThreads - 1) / kThreads;    // chunks per thread
  u32x4_t k[NC];
  u32x4_t v[NC];
};

// Per-thread element offsets of the 16-byte chunks a thread stages, relative to the
// subtile's first key (row stride rs); computed once per kernel.
template <int D>
struct KVOffsets {
  uint32_t off[KVRegs<D>::NC];
  __device__ __forceinline__ void init(size_t rs) {
    using R = KVRegs<D>;
#pragma unroll
    for (int i = 0; i < R::NC; ++i) {
      const int ci = min((int)threadIdx.x + i * kThreads, KN * R::CPR - 1);
      off[i] = (uint32_t)((ci / R::CPR) * rs + (ci % R::CPR) * 8);
    }
  }
};

// A full subtile: kp/vp point at its first key.
template <int D>
__device__ __forceinline__ void kv_load(KVRegs<D>& r, const KVOffsets<D>& o,
                                        const uint16_t* __restrict__ kp,
                                        const uint16_t* __restrict__ vp) {
#pragma unroll
  for (int i = 0; i < KVRegs<D>::NC; ++i) {
    r.k[i] = *reinterpret_cast<const u32x4_t*>(kp + o.off[i]);
    r.v[i] = *reinterpret_cast<const u32x4_t*>(vp + o.off[i]);
  }
}

// A partial subtile of nvalid keys.  Rows past nvalid re-read row nvalid-1: those keys
// are masked (score -inf, p = 0), so their values only need to be finite.
template <int D>
__device__ __forceinline__ void kv_load_partial(KVRegs<D>& r, const uint16_t* __restrict__ kp,
                                                const uint16_t* __restrict__ vp, size_t rs,
                                                int nvalid) {
  using R = KVRegs<D>;
#pragma unroll
  for (int i = 0; i < R::NC; ++i) {
    const int ci = min((int)threadIdx.x + i * kThreads, KN * R::CPR - 1);
    const int key = min(ci / R::CPR, nvalid - 1), ch = ci % R::CPR;
    r.k[i] = *reinterpret_cast<const u32x4_t*>(kp + key * rs + ch * 8);
    r.v[i] = *reinterpret_cast<const u32x4_t*>(vp + key * rs + ch * 8);
  }
}

template <int D>
__device__ __forceinline__ void kv_fetch(KVRegs<D>& r, const KVOffsets<D>& o,
                                         const uint16_t* __restrict__ kp,
                                         const uint16_t* __restrict__ vp, size_t rs,
                                         int nvalid) {
  if (nvalid == KN) kv_load<D>(r, o, kp, vp);
  else kv_load_partial<D>(r, kp, vp, rs, nvalid);
}

// K and V rows as they are, into padded rows
template <int D>
__device__ __forceinline__ void kv_store(const KVRegs<D>& r, char* lk, char* lv) {
  using R = KVRegs<D>;
  using L = Lds<D>;
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < R::NC; ++i) {
    const int ci = tid + i * kThreads;
    const int key = ci / R::CPR, ch = ci % R::CPR;
    if (ci < KN * R::CPR) {
      *reinterpret_cast<u32x4_t*>(lk + key * L::KS + ch * 16) = r.k[i];
      *reinterpret_cast<u32x4_t*>(lv + key * L::VS + ch * 16) = r.v[i];
    }
  }
}

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

// ds_read_b64_tr_b16: within each group of 16 lanes, lane i receives element i%4 of
// the 8 bytes addressed by lanes 4j + i/4, j = 0..3.
__device__ __forceinline__ u32x2_t lds_read_tr16(const char* p) {
  const s16x4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(p));
  return __builtin_bit_cast(u32x2_t, r);
}

__device__ __forceinline__ float pair_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                  false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                  false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int D, int QT>
__device__ __forceinline__ void state_init(WaveState<D, QT>& st) {
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    st.m[qt] = -INFINITY;
    st.l[qt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) st.o[qt][dt][i] = 0.f;
  }
}

// 32 keys (half kk of a 64-key subtile staged in LDS) for every query row of the wave.
// MASK: key rows >= nkeys and keys > tpos (causal) score -inf.  Lazy rescale: the
// reference max m moves only when a row's max exceeds it by more than kTau (O and l are
// rescaled then), so p = exp2(s * scale * log2e - m) <= 2^kTau.
template <int D, int QT, bool MASK>
__device__ __forceinline__ void attend_half(WaveState<D, QT>& st, const char* lk,
                                            const char* lv, int kk, float sl, int nkeys,
                                            int kb, const int (&tpos)[QT]) {
  const int lane = threadIdx.x & 63, n = lane & 31, hf = lane >> 5;
  f32x16_t s[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt)
#pragma unroll
    for (int i = 0; i < 16; ++i) s[qt][i] = 0.f;
  // A = K rows kk*32 + n, dims 16*ks + 8*hf .. +7
  const char* kp = lk + (kk * 32 + n) * Lds<D>::KS + hf * 16;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    const bf16x8_t a = as_bf16x8(*reinterpret_cast<const u32x4_t*>(kp + ks * 32));
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) s[qt] = mfma32x32x16(a, st.q[qt][ks], s[qt]);
  }
  float mxs[QT];
  bool need = false;
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    if (MASK) {
      // key kb + kk*32 + (i/4)*8 + hf*4 + i%4 is live iff its row < nkeys and key <= tpos
      const int lim = min(nkeys - 1, tpos[qt] - kb) - kk * 32 - hf * 4;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if ((i >> 2) * 8 + (i & 3) > lim) s[qt][i] = -INFINITY;
    }
    float mx = s[qt][0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[qt][i]);
    mx = pair_max(mx);
    mxs[qt] = mx * sl;
    need |= mxs[qt] > st.m[qt] + kTau;
  }
  if (__ballot(need) != 0ull) {
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const float mnew = fmaxf(st.m[qt], mxs[qt]);
      const float alpha = (mnew == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(st.m[qt] - mnew);
      st.m[qt] = mnew;
      st.l[qt] *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) st.o[qt][dt][i] *= alpha;
    }
  }
  bf16x8_t pb[QT][2];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const float mref = (st.m[qt] == -INFINITY) ? 0.f : st.m[qt];
    // the row sum stays float32: summing the bf16-rounded p would cost up to 2^-9
    // relative in lse for rows that attend only a few keys
    float rs = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = __builtin_amdgcn_exp2f(fmaf(s[qt][i], sl, -mref));
      s[qt][i] = p;
      rs += p;
    }
    st.l[qt] += rs;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(s[qt][8 * h + 2 * e], s[qt][8 * h + 2 * e + 1]);
      pb[qt][h] = as_bf16x8(u32x4_t{w[0], w[1], w[2], w[3]});
    }
  }
  // P^T for MFMA k-step ks = 2*kk + h is the score registers 8h .. 8h+7 of this half:
  // lane (n, hf) holds keys 16ks + 8(e/4) + 4hf + e%4, e < 8.  The matching V^T operand
  // is two transpose reads: lanes 4j+q of each 16-lane group address row
  // 16ks + 4hf + j (+8 for the second read), dims d0 + 4q .. +3, where d0 = dt*32 +
  // 16*((lane/16)&1); lane i of the group then holds dim d0 + i of those four keys.
  const char* vp = lv + (4 * hf + ((lane & 15) >> 2)) * Lds<D>::VS +
                   (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int ks = 2 * kk + h;
      const u32x2_t lo = lds_read_tr16(vp + (16 * ks) * Lds<D>::VS + dt * 64);
      const u32x2_t hi = lds_read_tr16(vp + (16 * ks + 8) * Lds<D>::VS + dt * 64);
      const bf16x8_t a = as_bf16x8(u32x4_t{lo[0], lo[1], hi[0], hi[1]});
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) st.o[qt][dt] = mfma32x32x16(a, pb[qt][h], st.o[qt][dt]);
    }
  }
}

// Subtiles [i0, i1) of the key range starting at key_begin, staged through two LDS
// buffers: the next subtile's global loads are in flight while the current one is
// computed, then written to the other buffer; one barrier per subtile.  On entry the
// subtile i0 is already in buffer i0 & 1.
template <int D, int QT, bool MASK>
__device__ __forceinline__ void attend_subtiles(WaveState<D, QT>& st, char* lds,
                                                KVRegs<D>& r, const KVOffsets<D>& ko,
                                                const uint16_t* __restrict__ kbase,
                                                const uint16_t* __restrict__ vbase, size_t rs,
                                                int key_begin, int key_end, int i0, int i1,
                                                int nsub, float sl, bool active,
                                                const int (&tpos)[QT]) {
  constexpr int STAGE = Lds<D>::STAGE;
  constexpr int KB = Lds<D>::KBYTES;
  for (int i = i0; i < i1; ++i) {
    const int kb = key_begin + i * KN;
    const bool more = i + 1 < nsub;
    if (more)
      kv_fetch<D>(r, ko, kbase + (size_t)(kb + KN) * rs, vbase + (size_t)(kb + KN) * rs, rs,
                  min(KN, key_end - kb - KN));
    const char* cur = lds + (i & 1) * STAGE;
    if (active) {
      const int nvalid = min(KN, key_end - kb);
      attend_half<D, QT, MASK>(st, cur, cur + KB, 0, sl, nvalid, kb, tpos);
      attend_half<D, QT, MASK>(st, cur, cur + KB, 1, sl, nvalid, kb, tpos);
    }
    if (more) {
      char* nxt = lds + ((i + 1) & 1) * STAGE;
      kv_store<D>(r, nxt, nxt + KB);
    }
    __syncthreads();
  }
}

// The wave's rows over keys [key_begin, key_end) of one kv-head.  Subtiles whose last
// key exceeds diag_from (the smallest query position of the workgroup) or key_end need
// the mask; they come last and run in their own loop.
template <int D, int QT>
__device__ __forceinline__ void attend_range(WaveState<D, QT>& st, char* lds,
                                             const uint16_t* __restrict__ kbase,
                                             const uint16_t* __restrict__ vbase, size_t rs,
                                             int key_begin, int key_end, float sl,
                                             bool active, int diag_from, const int (&tpos)[QT]) {
  KVRegs<D> r;
  KVOffsets<D> ko;
  ko.init(rs);
  const int nsub = (key_end - key_begin + KN - 1) / KN;
  // subtile i is mask-free iff key_begin + (i+1)*KN <= min(key_end, diag_from + 1)
  const int lim = min(key_end, diag_from == 0x7fffffff ? key_end : diag_from + 1);
  const int nplain = max(0, min(nsub, (lim - key_begin) / KN));
  kv_fetch<D>(r, ko, kbase + (size_t)key_begin * rs, vbase + (size_t)key_begin * rs, rs,
              min(KN, key_end - key_begin));
  kv_store<D>(r, lds, lds + Lds<D>::KBYTES);
  __syncthreads();
  attend_subtiles<D, QT, false>(st, lds, r, ko, kbase, vbase, rs, key_begin, key_end, 0,
                                nplain, nsub, sl, active, tpos);
  attend_subtiles<D, QT, true>(st, lds, r, ko, kbase, vbase, rs, key_begin, key_end, nplain,
                               nsub, nsub, sl, active, tpos);
}

// normalise and store one query tile's partial (o fp32 [D], lse natural log)
template <int D, int QT>
__device__ __forceinline__ void store_partial(const WaveState<D, QT>& st, int qt, bool valid,
                                              float* __restrict__ po, float* __restrict__ pl) {
  const int lane = threadIdx.x & 63, hf = lane >> 5;
  const float ltot = pair_sum(st.l[qt]);
  if (!valid) return;
  const float inv = 1.f / ltot;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      f32x4_t w;
#pragma unroll
      for (int r = 0; r < 4; ++r) w[r] = st.o[qt][dt][ii * 4 + r] * inv;
      *reinterpret_cast<f32x4_t*>(po + dt * 32 + ii * 8 + hf * 4) = w;
    }
  if (hf == 0) *pl = (st.m[qt] + __log2f(ltot)) * 0.69314718055994530942f;
}

template <int D, int QT>
__device__ __forceinline__ void load_q(WaveState<D, QT>& st, int qt, const uint16_t* qrow,
                                       bool valid) {
  const int hf = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    u32x4_t x = {0u, 0u, 0u, 0u};
    if (valid) x = *reinterpret_cast<const u32x4_t*>(qrow + 16 * ks + 8 * hf);
    st.q[qt][ks] = as_bf16x8(x);
  }
}

// ---------------------------------------------------------------- history (a4)
// One workgroup = one tile of up to 4 * 32 * QT gathered rows of one list (b, g, j).
template <int D, int QT>
__global__ __launch_bounds__(kThreads, MOBA_ATTN_WPE) void attn_history_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, int T, int hq, int hkv, int block, int topk,
    float sl, int g0, int ng, int nb, const int4* __restrict__ tiles,
    const int32_t* __restrict__ tile_count, const uint32_t* __restrict__ entries,
    float* __restrict__ part_o, float* __restrict__ part_lse) {
  __shared__ __attribute__((aligned(16))) char lds[2 * Lds<D>::STAGE];
  const int tile_id = blockIdx.x;
  if (tile_id >= *tile_count) return;
  const int4 tl = tiles[tile_id];
  const int list = tl.x;
  const int j = list % nb, gi = (list / nb) % ng, b = list / (nb * ng);
  const int G = hq / hkv, g = g0 + gi;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, n = lane & 31;

  WaveState<D, QT> st;
  int tq[QT], hlq[QT], slq[QT], tpos[QT];
  bool vq[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int e = tl.y + (wave * QT + qt) * 32 + n;
    vq[qt] = e < tl.z;
    const uint32_t ent = vq[qt] ? entries[e] : 0u;
    slq[qt] = (int)(ent & 31u);
    const int rr = (int)(ent >> 5);
    tq[qt] = rr / G;
    hlq[qt] = rr % G;
    tpos[qt] = 0x7fffffff;    // history keys all precede the query
    const uint16_t* qrow = q + ((size_t)((size_t)b * T + tq[qt]) * hq + g * G + hlq[qt]) * D;
    load_q(st, qt, qrow, vq[qt]);
  }
  state_init(st);
  const size_t rs = (size_t)hkv * D;
  const uint16_t* kbase = k + ((size_t)b * T * hkv + g) * D;
  const uint16_t* vbase = v + ((size_t)b * T * hkv + g) * D;
  const int key_begin = j * block;
  attend_range<D, QT>(st, lds, kbase, vbase, rs, key_begin, key_begin + block, sl, true,
                      0x7fffffff, tpos);
  const int ngq = ng * G;
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const size_t prow = ((size_t)(b * ngq + gi * G + hlq[qt]) * T + tq[qt]) * topk + slq[qt];
    store_partial(st, qt, vq[qt], part_o + prow * D, part_lse + prow);
  }
}

// ---------------------------------------------------------------- current (a5)
// One workgroup = 32*QT consecutive tokens of block c; its waves are the query heads
// of kv-head g (in rounds of four), so all four share every staged K/V subtile.
// Tiles run from the end of the block backwards: the longest ones start first.
template <int D, int QT>
__global__ __launch_bounds__(kThreads, MOBA_ATTN_WPE) void attn_current_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, int T, int hq, int hkv, int block, int topk,
    float sl, int g0, int ng, float* __restrict__ part_o, float* __restrict__ part_lse) {
  __shared__ __attribute__((aligned(16))) char lds[2 * Lds<D>::STAGE];
  constexpr int TT = 32 * QT;
  const int c = blockIdx.y;
  const int gi = blockIdx.z % ng, b = blockIdx.z / ng;
  const int G = hq / hkv, g = g0 + gi;
  const int x = gridDim.x - 1 - blockIdx.x;
  const int t0 = c * block + x * TT;
  const int t_end = min(t0 + TT, (c + 1) * block);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, n = lane & 31;
  const size_t rs = (size_t)hkv * D;
  const uint16_t* kbase = k + ((size_t)b * T * hkv + g) * D;
  const uint16_t* vbase = v + ((size_t)b * T * hkv + g) * D;
  const int ngq = ng * G;
  for (int round = 0; round * 4 < G; ++round) {
    const int hl = round * 4 + wave;
    const bool active = hl < G;
    WaveState<D, QT> st;
    int tpos[QT];
    bool vq[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      tpos[qt] = t0 + qt * 32 + n;
      vq[qt] = active && tpos[qt] < t_end;
      const uint16_t* qrow = q + ((size_t)((size_t)b * T + (vq[qt] ? tpos[qt] : 0)) * hq +
                                  g * G + (active ? hl : 0)) * D;
      load_q(st, qt, qrow, vq[qt]);
    }
    state_init(st);
    attend_range<D, QT>(st, lds, kbase, vbase, rs, c * block, t_end, sl, active, t0, tpos);
    if (active) {
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        const size_t prow =
            ((size_t)(b * ngq + gi * G + hl) * T + (vq[qt] ? tpos[qt] : 0)) * topk + (topk - 1);
        store_partial(st, qt, vq[qt], part_o + prow * D, part_lse + prow);
      }
    }
  }
}

// ---------------------------------------------------------------- merge (a5)
template <int D>
__global__ __launch_bounds__(kThreads) void merge_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_lse, int bsz, int T,
    int hq, int hkv, int block, int topk, int g0, int ng, uint16_t* __restrict__ out,
    float* __restrict__ lse) {
  constexpr int TPR = D / 4;
  constexpr int RPB = kThreads / TPR;
  const int G = hq / hkv, ngq = ng * G;
  const size_t row = (size_t)blockIdx.x * RPB + threadIdx.x / TPR;
  const size_t nrows = (size_t)bsz * ngq * T;
  if (row >= nrows) return;
  const int sub = threadIdx.x % TPR;
  const int t = (int)(row % T);
  const int hc = (int)((row / T) % ngq);
  const int b = (int)(row / ((size_t)T * ngq));
  const int h = g0 * G + hc;
  const int KH = topk - 1;
  const int nh = min(t / block, KH);
  const float* pl = part_lse + row * topk;
  const float* po = part_o + row * topk * D + 4 * sub;
  float mx = pl[KH];
  for (int s = 0; s < nh; ++s) mx = fmaxf(mx, pl[s]);
  float den = expf(pl[KH] - mx);
  for (int s = 0; s < nh; ++s) den += expf(pl[s] - mx);
  const float L = mx + logf(den);
  f32x4_t acc;
  {
    const float w = expf(pl[KH] - L);
    const f32x4_t x = *reinterpret_cast<const f32x4_t*>(po + (size_t)KH * D);
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] = w * x[r];
  }
  for (int s = 0; s < nh; ++s) {
    const float w = expf(pl[s] - L);
    const f32x4_t x = *reinterpret_cast<const f32x4_t*>(po + (size_t)s * D);
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] += w * x[r];
  }
  u32x2_t pk;
  pk[0] = f32_to_bf16_rne(acc[0]) | (f32_to_bf16_rne(acc[1]) << 16);
  pk[1] = f32_to_bf16_rne(acc[2]) | (f32_to_bf16_rne(acc[3]) << 16);
  *reinterpret_cast<u32x2_t*>(out + ((size_t)((size_t)b * T + t) * hq + h) * D + 4 * sub) = pk;
  if (sub == 0) lse[((size_t)b * hq + h) * T + t] = L;
}

// ---------------------------------------------------------------- launchers
constexpr int kQT = MOBA_ATTN_QT;
int history_tile_rows() { return 4 * 32 * kQT; }

hipError_t launch_attn_history(const Shape& s, const uint16_t* q, const uint16_t* k,
                               const uint16_t* v, float scale, int g0, int ng,
                               const int4* tiles, const int32_t* tile_count,
                               int max_tiles, const uint32_t* entries, float* part_o,
                               float* part_lse, hipStream_t st) {
  if (max_tiles <= 0) return hipSuccess;
  const float sl = scale * 1.4426950408889634f;
  if (s.d == 128)
    hipLaunchKernelGGL((attn_history_kernel<128, kQT>), dim3(max_tiles), dim3(kThreads), 0,
                       st, q, k, v, s.T, s.hq, s.hkv, s.block, s.topk, sl, g0, ng, s.nb(),
                       tiles, tile_count, entries, part_o, part_lse);
  else
    hipLaunchKernelGGL((attn_history_kernel<64, kQT>), dim3(max_tiles), dim3(kThreads), 0,
                       st, q, k, v, s.T, s.hq, s.hkv, s.block, s.topk, sl, g0, ng, s.nb(),
                       tiles, tile_count, entries, part_o, part_lse);
  return hipGetLastError();
}

hipError_t launch_attn_current(const Shape& s, const uint16_t* q, const uint16_t* k,
                               const uint16_t* v, float scale, int g0, int ng,
                               float* part_o, float* part_lse, hipStream_t st) {
  const float sl = scale * 1.4426950408889634f;
  constexpr int TT = 32 * kQT;
  dim3 grid((s.block + TT - 1) / TT, s.nb(), s.b * ng);
  if (s.d == 128)
    hipLaunchKernelGGL((attn_current_kernel<128, kQT>), grid, dim3(kThreads), 0, st, q, k,
                       v, s.T, s.hq, s.hkv, s.block, s.topk, sl, g0, ng, part_o, part_lse);
  else
    hipLaunchKernelGGL((attn_current_kernel<64, kQT>), grid, dim3(kThreads), 0, st, q, k,
                       v, s.T, s.hq, s.hkv, s.block, s.topk, sl, g0, ng, part_o, part_lse);
  return hipGetLastError();
}

hipError_t launch_merge(const Shape& s, int g0, int ng, const float* part_o,
                        const float* part_lse, uint16_t* out, float* lse, hipStream_t st) {
  const size_t rows = (size_t)s.b * ng * s.G() * s.T;
  const int rpb = kThreads / (s.d / 4);
  dim3 grid((unsigned)((rows + rpb - 1) / rpb));
  if (s.d == 128)
    hipLaunchKernelGGL((merge_kernel<128>), grid, dim3(kThreads), 0, st, part_o, part_lse,
                       s.b, s.T, s.hq, s.hkv, s.block, s.topk, g0, ng, out, lse);
  else
    hipLaunchKernelGGL((merge_kernel<64>), grid, dim3(kThreads), 0, st, part_o, part_lse,
                       s.b, s.T, s.hq, s.hkv, s.block, s.topk, g0, ng, out, lse);
  return hipGetLastError();
}

}  // namespace moba
