// Block-sparse attention: history blocks (gather-and-densify) write (o, lse) partials;
// the causal current block is computed last and its epilogue merges the partials by
// log-sum-exp into the output.
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
// K and V tiles are row-major in LDS with padded rows (K: +16 B, V: +64 B), which
// spreads the MFMA operand reads over all banks and lets every read use a per-lane
// base address plus an immediate offset.
// Online softmax in the log2 domain (scale * log2(e) folded into one FMA).
#include <algorithm>

#include "moba_internal.h"

namespace moba {

// query rows per wavefront = 32 * QT; waves per SIMD the compiler budgets for
#ifndef MOBA_ATTN_QT
#define MOBA_ATTN_QT 1
#endif
#ifndef MOBA_ATTN_WPE
#define MOBA_ATTN_WPE 2
#endif
// wavefronts per attention workgroup; every staged K/V subtile serves all of them
#ifndef MOBA_ATTN_NW
#define MOBA_ATTN_NW 8
#endif
constexpr int kAttnWaves = MOBA_ATTN_NW;
static_assert(kAttnWaves % 2 == 0, "the walker runs two wave groups");
constexpr int kAttnThreads = 64 * kAttnWaves;

#ifndef MOBA_ATTN_KN
#define MOBA_ATTN_KN 64
#endif
constexpr int KN = MOBA_ATTN_KN;  // keys per LDS subtile (a multiple of 32)
constexpr int NH = KN / 32;       // 32-key halves of a subtile (one MFMA row block each)
static_assert(KN % 32 == 0, "subtiles hold whole 32-key MFMA blocks");
constexpr float kTau = 8.f;     // lazy rescale: the reference max may lag by 2^8

template <int D>
struct Lds {
  static constexpr int KS = D * 2 + 16;          // K row stride (bytes)
  // V row stride: a transpose read serves 32 lanes = 4 key rows x 64 bytes per pass;
  // a stride of 16 dwords (mod 64 banks) puts those rows on disjoint banks
  static constexpr int VS = D * 2 + 64;          // V row stride (bytes)
  static constexpr int KBYTES = KN * KS;
  static constexpr int VBYTES = KN * VS;
  static constexpr int NBUF = 3;                 // K and V subtile buffers each
  static constexpr int TOTAL = NBUF * (KBYTES + VBYTES);
};

template <int D, int QT>
struct WaveState {
  bf16x8_t q[QT][D / 16];
  f32x16_t o[QT][D / 32];
  float m[QT], l[QT];
};

// One KN-key subtile of K (or V) in flight through registers (global -> regs -> LDS).
template <int D>
struct TileRegs {
  static constexpr int CPR = D / 8;                                  // 16 B chunks per row
  static constexpr int NC = (KN * CPR + kAttnThreads - 1) / kAttnThreads;    // chunks per thread
  u32x4_t c[NC];
};

// Per-thread element offsets of the chunks a thread stages, relative to the subtile's
// first key (row stride rs); computed once per kernel.
template <int D>
struct TileOffsets {
  uint32_t off[TileRegs<D>::NC];
  __device__ __forceinline__ void init(size_t rs) {
    using R = TileRegs<D>;
#pragma unroll
    for (int i = 0; i < R::NC; ++i) {
      const int ci = min((int)threadIdx.x + i * kAttnThreads, KN * R::CPR - 1);
      off[i] = (uint32_t)((ci / R::CPR) * rs + (ci % R::CPR) * 8);
    }
  }
};

// p points at the subtile's first key (a wave-uniform address).  The loads go through
// a buffer descriptor covering exactly the nvalid rows of the subtile: the 32-bit
// offsets need no 64-bit address arithmetic, and the rows past a partial subtile's
// end read as zeros (those keys are masked, so any finite value would do).
template <int D>
__device__ __forceinline__ void tile_load(TileRegs<D>& r, const TileOffsets<D>& o,
                                          const uint16_t* __restrict__ p, size_t rs,
                                          int nvalid) {
  using R = TileRegs<D>;
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(p), (short)0, (int)(nvalid * rs * sizeof(uint16_t)), 0x00020000);
#pragma unroll
  for (int i = 0; i < R::NC; ++i) {
    const auto x = __builtin_amdgcn_raw_buffer_load_b128(rsrc, (int)(o.off[i] * 2), 0, 0);
    r.c[i] = __builtin_bit_cast(u32x4_t, x);
  }
}

// The same through a descriptor made once for a whole key range, the subtile selected
// by the scalar byte offset soff; rows past the range's end read as zeros.
template <int D>
__device__ __forceinline__ void tile_load_rs(TileRegs<D>& r, const TileOffsets<D>& o,
                                             __amdgpu_buffer_rsrc_t rsrc, int soff) {
  using R = TileRegs<D>;
#pragma unroll
  for (int i = 0; i < R::NC; ++i) {
    const auto x = __builtin_amdgcn_raw_buffer_load_b128(rsrc, (int)(o.off[i] * 2), soff, 0);
    r.c[i] = __builtin_bit_cast(u32x4_t, x);
  }
}

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef __attribute__((address_space(3))) char lds_char;   // a byte of LDS

// ds_read_b64_tr_b16: within each group of 16 lanes, lane i receives element i%4 of
// the 8 bytes addressed by lanes 4j + i/4, j = 0..3.
__device__ __forceinline__ u32x2_t lds_read_tr16(const char* p) {
  const s16x4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(p));
  return __builtin_bit_cast(u32x2_t, r);
}
__device__ __forceinline__ u32x2_t lds_read_tr16(const lds_char* p) {
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

// Key-range walker.  Per KN-key subtile i a wavefront runs two phases:
//   A(i)   the QK^T MFMAs of subtile i+1 next to the exp/sum/pack of subtile i;
//   B(i)   the PV MFMAs of subtile i next to the mask and row max of subtile i+1, then
//          the lazy-rescale decision;
// after a phase P (QK^T of subtile 0, its mask and row max).  The workgroup's waves form
// two groups (the two waves that share a SIMD are in different groups), and one
// barrier per subtile ends an interval:
//   group 0:  P | A(0) B(0) | A(1) B(1) | ... | A(n-1) B(n-1)
//   group 1:  P A(0) | B(0) A(1) | B(1) A(2) | ... | B(n-1)
// so in every interval one wave of a SIMD starts in an exp-heavy phase while the other
// starts in an MFMA/LDS-heavy one, and the two swap half-way without a barrier.
// LDS holds three K and three V subtile buffers (subtile i in buffer i % 3).  Interval
// n reads K(n), K(n+1), V(n-1) and V(n); it stages K(n+2) and V(n+1) from registers
// loaded in interval n-1, so a subtile is visible an interval before it is first read,
// and a buffer is rewritten only after the interval that read its previous subtile.
// The operand reads run PF MFMAs ahead as one stream over a wave's phases: the last
// slots of a phase read the first operands of the next one, across the barrier too,
// so no phase starts by waiting on the LDS.  Staging past the last subtile re-stages
// the last subtile into buffers nobody reads again.
// CHAIN: the walk runs over the subtiles of all of a persistent workgroup's tiles one
// after the other (virtual subtile i is subtile i % nsub of the workgroup's tile
// i / nsub), so the next tile's first K/V subtiles are staged, and its query rows
// loaded, while the current tile finishes: see attn_history_chain_kernel.
template <int D, int QT, bool CHAIN = false>
struct Walker {
  using L = Lds<D>;
  static constexpr int KSTEPS = D / 16;            // MFMA k-steps over the head dim
  static constexpr int NQK = NH * KSTEPS;          // QK^T MFMAs per query tile
  static constexpr int NPV = (KN / 16) * (D / 32); // PV MFMAs per query tile
#ifndef MOBA_ATTN_PF
#define MOBA_ATTN_PF 4
#endif
  static constexpr int PF = MOBA_ATTN_PF;          // operand reads in flight
  static_assert(NQK % PF == 0 && NPV % PF == 0, "every phase starts at the ring's head");
  static constexpr int NC = TileRegs<D>::NC;
#ifndef MOBA_ATTN_SS
#define MOBA_ATTN_SS 2
#endif
  static constexpr int SS = MOBA_ATTN_SS;          // first staging slot of an interval
  static_assert(SS + 2 * NC < NQK && SS + 2 * NC < NPV, "staging fits in one phase");

  using Scores = f32x16_t[NH][QT];
  using POps = bf16x8_t[QT][KN / 16];
  using Ops = u32x4_t[PF];
  lds_char* lds;
  const uint16_t* kbase;
  const uint16_t* vbase;
  size_t rs;
  int key_begin, key_end, nsub, diag_from;
  float sl;
  int grp;                     // 0: A before B in an interval, 1: B before A
  uint32_t kl, vl;             // the lane's byte offsets of its K and V operand reads
  TileOffsets<D> to;
  TileRegs<D> kst, vst, pre;   // staging registers (pre: K(1) in the prologue only)
  // one buffer descriptor each for the K and V rows of [key_begin, key_end) (not CHAIN)
  __amdgpu_buffer_rsrc_t kdesc, vdesc;
  // CHAIN:
  //  * the tile list, and the workgroup's tiles taken from a queue: tq[s % 4] holds the
  //    index of its tile s for the tiles in use (s = it .. it + 2); queue is the
  //    counter, qpend thread 0's request in flight; ntiles is the list's tile count;
  //  * ntw, the workgroup's tile count once known, and ntiles before (a bound; the
  //    launcher keeps nsub * ntiles below 2^30, so len() cannot overflow);
  //  * what locates a tile's block (key_end - key_begin keys, a multiple of KN, so no
  //    subtile is masked);
  //  * the walk's position (subtile im of tile it), and the two staging streams' next
  //    subtile (local index, tile, the tile's first-key offset).
  const int4* tiles;
  __attribute__((address_space(3))) int* tq;
  int* queue;
  int qpend;
  int ntiles, ntw, nb, ng, g0, hkv;
  SeqMap sq;
  int im, it;
  int kt_l, kt_t, vt_l, vt_t;
  size_t kt_off, vt_off;
  __device__ __forceinline__ int len() const { return CHAIN ? nsub * ntw : nsub; }
  // index in the tile list of the workgroup's tile s (the last tile past the end)
  __device__ __forceinline__ int tile_of(int s) const {
    return __builtin_amdgcn_readfirstlane(tq[min(s, ntw - 1) & 3]);
  }
  // element offset of the first key of the block of the workgroup's tile s (the last
  // tile past the end)
  __device__ __forceinline__ size_t tile_keys(int s) const {
    const int list = tiles[tile_of(s)].x;
    const int j = list % nb, gi = (list / nb) % ng, b = list / (nb * ng);
    return (((size_t)sq.tok0(b) + (size_t)j * (key_end - key_begin)) * hkv + g0 + gi) * D;
  }
  // CHAIN: load a staging stream's next subtile (the last subtile of the last tile once
  // past the end), then advance the stream by one subtile
  __device__ __forceinline__ void load_stream(TileRegs<D>& r, bool isv, int& l, int& t,
                                              size_t& off) {
    const int lc = t < ntw ? l : nsub - 1;
    tile_load<D>(r, to, (isv ? vbase : kbase) + off + (size_t)lc * KN * rs, rs, KN);
    if (++l == nsub) {
      l = 0;
      ++t;
      off = tile_keys(t);
    }
  }

  // The buffer offsets pass through an empty asm so that the compiler adds them to the
  // lane's base address at run time: folded into the reads' 16-bit immediate offsets,
  // the upper buffers' constants overflow it, and the compiler then keeps one address
  // register per (buffer, read) live across the whole walk.
  __device__ __forceinline__ lds_char* kbuf(int i) const {
    int off = (i % L::NBUF) * L::KBYTES;
    asm("" : "+s"(off));
    return lds + off;
  }
  __device__ __forceinline__ lds_char* vbuf(int i) const {
    int off = L::NBUF * L::KBYTES + (i % L::NBUF) * L::VBYTES;
    asm("" : "+s"(off));
    return lds + off;
  }
  __device__ __forceinline__ int kb(int i) const {
    return key_begin + (CHAIN ? i % nsub : i) * KN;
  }
  __device__ __forceinline__ int nvalid(int i) const { return min(KN, key_end - kb(i)); }
  __device__ __forceinline__ bool masked(int i) const {
    if constexpr (CHAIN) return false;
    return kb(i) + KN > key_end || kb(i) + KN - 1 > diag_from;
  }
  // global -> registers: subtile i (the last one past the end) of K (isv false) or V
  __device__ __forceinline__ void load_sub(TileRegs<D>& r, bool isv, int i) {
    if constexpr (!CHAIN) {
      const int t = min(i, nsub - 1);
      tile_load_rs<D>(r, to, isv ? vdesc : kdesc, t * (int)(KN * rs * sizeof(uint16_t)));
      return;
    }
    const int t = min(i, len() - 1);
    const uint16_t* p;
    if constexpr (CHAIN) p = (isv ? vbase : kbase) + tile_keys(t / nsub) + (size_t)(kb(t) - key_begin) * rs;
    else p = (isv ? vbase : kbase) + (size_t)kb(t) * rs;
    tile_load<D>(r, to, p, rs, nvalid(t));
  }
  // registers -> LDS: chunk c of a subtile into a buffer of row stride STRIDE
  template <int STRIDE>
  __device__ __forceinline__ static void store_chunk(const TileRegs<D>& r, int c, lds_char* buf) {
    constexpr bool kAllThreads = (KN * TileRegs<D>::CPR) % kAttnThreads == 0;
    const int ci = threadIdx.x + c * kAttnThreads;
    if (kAllThreads || ci < KN * TileRegs<D>::CPR)
      *reinterpret_cast<__attribute__((address_space(3))) u32x4_t*>(buf + (ci / TileRegs<D>::CPR) * STRIDE +
                                  (ci % TileRegs<D>::CPR) * 16) = r.c[c];
  }
  // slot j of interval n's first phase: K(n+2) and V(n+1) go from the registers into
  // LDS chunk by chunk, then K(n+3) and V(n+2) are loaded into the same registers
  __device__ __forceinline__ void stage_slot(int j, int n) {
    const int s = j - SS;
    if (s >= 0 && s < 2 * NC) {
      if (s & 1) store_chunk<L::VS>(vst, s >> 1, vbuf(n + 1));
      else store_chunk<L::KS>(kst, s >> 1, kbuf(n + 2));
    } else if (s == 2 * NC) {
      if constexpr (CHAIN) {
        load_stream(kst, false, kt_l, kt_t, kt_off);
        load_stream(vst, true, vt_l, vt_t, vt_off);
      } else {
        load_sub(kst, false, n + 3);
        load_sub(vst, true, n + 2);
      }
    }
  }

  // QK^T MFMA j: 32-key half qk_kk(j), k-step qk_ks(j) (the NH accumulator chains
  // alternate, so consecutive MFMAs are independent)
  __device__ __forceinline__ static constexpr int qk_kk(int j) { return j % NH; }
  __device__ __forceinline__ static constexpr int qk_ks(int j) { return j / NH; }
  __device__ __forceinline__ static int k_off(int j) {
    return qk_kk(j) * 32 * L::KS + qk_ks(j) * 32;
  }
  // K operand of QK^T MFMA j of a subtile in buffer kbufp
  __device__ __forceinline__ u32x4_t kread(const lds_char* kbufp, int j) const {
    return *reinterpret_cast<const __attribute__((address_space(3))) u32x4_t*>(kbufp + kl + k_off(j));
  }
  // V^T operand of PV MFMA j of a subtile in buffer vbufp
  __device__ __forceinline__ u32x4_t vread(const lds_char* vbufp, int j) const {
    const int ks = j / (D / 32), dt = j % (D / 32);
    const lds_char* p = vbufp + vl + (16 * ks) * L::VS + dt * 64;
    const u32x2_t lo = lds_read_tr16(p);
    const u32x2_t hi = lds_read_tr16(p + 8 * L::VS);
    return u32x4_t{lo[0], lo[1], hi[0], hi[1]};
  }
  // operand j of the next phase: NX = 1 its K, 2 its V
  template <int NX>
  __device__ __forceinline__ u32x4_t nread(const lds_char* bufp, int j) const {
    return NX == 1 ? kread(bufp, j) : vread(bufp, j);
  }

  __device__ __forceinline__ void mask_scores(Scores& s, int i, const int (&tpos)[QT]) const {
    const int hf = (threadIdx.x & 63) >> 5;
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
#pragma unroll
      for (int kk = 0; kk < NH; ++kk) {
        const int lim = min(nvalid(i) - 1, tpos[qt] - kb(i)) - kk * 32 - hf * 4;
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if ((e >> 2) * 8 + (e & 3) > lim) s[kk][qt][e] = -INFINITY;
      }
  }

  __device__ __forceinline__ void rescale(WaveState<D, QT>& st, const float (&mxs)[QT]) {
    bool need = false;
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) need |= mxs[qt] > st.m[qt] + kTau;
    if (__ballot(need) != 0ull) {
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        const float mnew = fmaxf(st.m[qt], mxs[qt]);
        const float alpha =
            (mnew == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(st.m[qt] - mnew);
        st.m[qt] = mnew;
        st.l[qt] *= alpha;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int e = 0; e < 16; ++e) st.o[qt][dt][e] *= alpha;
      }
    }
  }

  // mask, row max and rescale of subtile i's scores, all at once (after phase P)
  __device__ __forceinline__ void max_all(WaveState<D, QT>& st, Scores& s, int i,
                                          const int (&tpos)[QT]) {
    if (masked(i)) mask_scores(s, i, tpos);
    float mxs[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      float mx = -INFINITY;
#pragma unroll
      for (int kk = 0; kk < NH; ++kk)
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[kk][qt][e]);
      mxs[qt] = pair_max(mx) * sl;
    }
    rescale(st, mxs);
  }

  // Phase A(i) (EXP) or P (!EXP): QK^T of the subtile in buffer kq into nxt (when NEXT)
  // next to the exp/sum/pack of cur into pb.  ops holds the first PF K operands; the
  // last PF slots read the next phase's first operands from buffer nb (NX = 1: K,
  // 2: V; 0: ops is left as it is).  With STAGE the phase carries interval n's staging.
  template <bool NEXT, bool EXP, int NX, bool STAGE>
  __device__ __forceinline__ void phase_a(WaveState<D, QT>& st, const Scores& cur,
                                          Scores& nxt, POps& pb, Ops& ops, const lds_char* kq,
                                          const lds_char* nb, int n) {
    constexpr int EPS = 16 * NH / NQK;  // exp elements per slot and query tile
    static_assert(EPS * NQK == 16 * NH && 8 % EPS == 0, "the exps split evenly over slots");
    static_assert(NEXT || NX == 0, "a phase without MFMAs reads no operands");
    float mref[QT], rsum[QT], p[QT][16 * NH];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      mref[qt] = (st.m[qt] == -INFINITY) ? 0.f : st.m[qt];
      rsum[qt] = 0.f;
    }
    const f32x16_t zero = {};
#pragma unroll
    for (int j = 0; j < NQK; ++j) {
      if (NEXT) {
        const int kk = qk_kk(j), ks = qk_ks(j);
        const bf16x8_t a = as_bf16x8(ops[j % PF]);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
          nxt[kk][qt] = mfma32x32x16(a, st.q[qt][ks], ks == 0 ? zero : nxt[kk][qt]);
        if (j + PF < NQK) ops[j % PF] = kread(kq, j + PF);
        else if (NX != 0) ops[j % PF] = nread<NX>(nb, j + PF - NQK);
      }
      if (EXP) {
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
#pragma unroll
          for (int e = 0; e < EPS; ++e) {
            const int x = j * EPS + e;
            p[qt][x] = __builtin_amdgcn_exp2f(fmaf(cur[x >> 4][qt][x & 15], sl, -mref[qt]));
            rsum[qt] += p[qt][x];
          }
          // P^T operand of k-step ks = score registers 8*(ks%2) .. +7 of half ks/2,
          // packed as soon as its 8 values exist
          if (((j + 1) * EPS) % 8 == 0) {
            const int ks = (j + 1) * EPS / 8 - 1;
            uint32_t w[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
              w[e] = pack_bf16x2(p[qt][8 * ks + 2 * e], p[qt][8 * ks + 2 * e + 1]);
            pb[qt][ks] = as_bf16x8(u32x4_t{w[0], w[1], w[2], w[3]});
            // keep this slice in this slot: without the pin the compiler sinks the
            // whole exp/pack work past the barrier into phase B, next to its use
            asm volatile("" : "+v"(pb[qt][ks]));
          }
        }
      }
      if (STAGE) stage_slot(j, n);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (EXP) {
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        asm volatile("" : "+v"(rsum[qt]));
        st.l[qt] += rsum[qt];
      }
    }
  }

  // Phase B(i): O^T += V^T P^T for the subtile in buffer vq next to the mask and row max
  // of nxt (subtile i+1, when NEXT), then the rescale decision.  Operand stream and
  // staging as in phase_a.
  template <bool NEXT, int NX, bool STAGE, typename Post>
  __device__ __forceinline__ void phase_b(WaveState<D, QT>& st, Scores& nxt, const POps& pb,
                                          Ops& ops, const lds_char* vq, const lds_char* nb,
                                          int i, int n, const int (&tpos)[QT], Post&& post) {
    if (NEXT && masked(i + 1)) mask_scores(nxt, i + 1, tpos);
    constexpr int MPS = 16 * NH / NPV;  // max elements per slot and query tile
    static_assert(MPS * NPV == 16 * NH, "the row max splits evenly over the PV slots");
    float mx[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) mx[qt] = -INFINITY;
#pragma unroll
    for (int j = 0; j < NPV; ++j) {
      const int ks = j / (D / 32), dt = j % (D / 32);
      const bf16x8_t a = as_bf16x8(ops[j % PF]);
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) st.o[qt][dt] = mfma32x32x16(a, pb[qt][ks], st.o[qt][dt]);
      if (j + PF < NPV) ops[j % PF] = vread(vq, j + PF);
      else if (NX != 0) ops[j % PF] = nread<NX>(nb, j + PF - NPV);
      if (NEXT) {
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
#pragma unroll
          for (int e = 0; e < MPS; ++e) {
            const int x = j * MPS + e;
            mx[qt] = fmaxf(mx[qt], nxt[x >> 4][qt][x & 15]);
          }
      }
      if (STAGE) stage_slot(j, n);
      __builtin_amdgcn_sched_barrier(0);
    }
    float mxs[QT];
    if (NEXT) {
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) mxs[qt] = pair_max(mx[qt]) * sl;
    }
    post();
    if (NEXT) rescale(st, mxs);
  }

  // Subtile i: A(i), then B(i).  Both groups run this same code; group 1's barrier
  // falls between the two phases, group 0's after B.  A(i) carries the staging of
  // interval i + 1 - grp.  KIND 0: i + 2 < len, 1: i = len - 2, 2: i = len - 1.
  // CHAIN: when A(i+1) starts the next tile (its QK^T is that tile's first), B(i)
  // first loads the tile's query rows (next_q); when B(i) ends a tile, `bound` stores
  // it and resets the state after the PV MFMAs, before the rescale that starts the next.
  template <int KIND, typename NextQ, typename Bound>
  __device__ __forceinline__ void iter(WaveState<D, QT>& st, Scores& cur, Scores& nxt,
                                       POps& pb, Ops& ops, int i, const int (&tpos)[QT],
                                       NextQ&& next_q, Bound&& bound) {
    // B(i) carries the staging of interval i + 1, in which it runs for both groups.
    // A wavefront raises its priority for the exp-heavy phase A: the two waves of a
    // SIMD then get through an interval at the same pace instead of the older one
    // finishing its phases early and idling at the barrier while the other runs alone.
    const int n = i + 1;
    __builtin_amdgcn_s_setprio(1);
    if (KIND < 2) phase_a<true, true, 2, false>(st, cur, nxt, pb, ops, kbuf(i + 1), vbuf(i), n);
    else phase_a<false, true, 0, false>(st, cur, nxt, pb, ops, nullptr, nullptr, n);
    __builtin_amdgcn_s_setprio(0);
    if (grp) __syncthreads();
    if constexpr (CHAIN && KIND == 0) {
      // the queue, two tiles ahead: thread 0 takes tile it + 2 at subtile 0 and
      // publishes it at subtile 1; every wave reads it at subtile 2, after a barrier
      // that follows the write for both groups (tiles have at least four subtiles)
      if (threadIdx.x == 0) {
        if (im == 0) qpend = atomicAdd(queue, 1);
        else if (im == 1) tq[(it + 2) & 3] = (int)gridDim.x + qpend;
      }
      // (a select, not a branch: as a branch next to the divergent one above, this
      // compiler fails with an illegal VGPR to SGPR copy)
      const int t2 = __builtin_amdgcn_readfirstlane(tq[(it + 2) & 3]);
      ntw = (im == 2 && t2 >= ntiles) ? min(ntw, it + 2) : ntw;
      if (im == nsub - 2) next_q(it + 1);
    }
    auto post = [&] {
      if constexpr (CHAIN && KIND == 0) {
        if (im == nsub - 1) bound(it);
      }
    };
    if (KIND == 0)
      phase_b<true, 1, true>(st, nxt, pb, ops, vbuf(i), kbuf(i + 2), i, n, tpos, post);
    else if (KIND == 1)
      phase_b<true, 2, true>(st, nxt, pb, ops, vbuf(i), vbuf(i + 1), i, n, tpos, post);
    else
      phase_b<false, 0, true>(st, nxt, pb, ops, vbuf(i), nullptr, i, n, tpos, post);
    if (!grp) __syncthreads();
    if constexpr (CHAIN) {
      if (++im == nsub) {
        im = 0;
        ++it;
      }
    }
  }

  __device__ __forceinline__ static void copy_scores(Scores& dst, const Scores& src) {
#pragma unroll
    for (int kk = 0; kk < NH; ++kk)
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) dst[kk][qt] = src[kk][qt];
  }

  // The first loads, which depend on nothing the caller computes, issued before the
  // caller's query loads so that their latencies overlap: K(0), K(1) and V(0).
  __device__ __forceinline__ void begin() {
    to.init(rs);
    nsub = (key_end - key_begin + KN - 1) / KN;
    const int lane = threadIdx.x & 63, hf = lane >> 5;
    kl = (uint32_t)((lane & 31) * L::KS + hf * 16);
    vl = (uint32_t)((4 * hf + ((lane & 15) >> 2)) * L::VS +
                    (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2);
    if constexpr (CHAIN) {
      // tile 0's first subtiles (a tile has at least four); the streams then go on
      // from K(3) and V(2)
      im = 0;
      it = 0;
      kt_off = vt_off = tile_keys(0);
      kt_l = 0;
      kt_t = 0;
      vt_l = 0;
      vt_t = 0;
      load_stream(kst, false, kt_l, kt_t, kt_off);
      load_stream(pre, false, kt_l, kt_t, kt_off);
      load_stream(vst, true, vt_l, vt_t, vt_off);
    } else {
      const int bytes = (int)((size_t)(key_end - key_begin) * rs * sizeof(uint16_t));
      kdesc = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(kbase + (size_t)key_begin * rs), (short)0, bytes, 0x00020000);
      vdesc = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(vbase + (size_t)key_begin * rs), (short)0, bytes, 0x00020000);
      load_sub(kst, false, 0);
      load_sub(pre, false, 1);
      load_sub(vst, true, 0);
    }
  }

  // CHAIN: the walk's length (len()) becomes known from the queue while it runs, at
  // least a tile before its end.
  template <typename NextQ, typename Bound>
  __device__ __forceinline__ void run(WaveState<D, QT>& st, const int (&tpos)[QT],
                                      NextQ&& next_q, Bound&& bound) {
    // prologue: K(0), K(1) and V(0) into LDS, then the registers that interval 0
    // stages (K(2), V(1))
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      store_chunk<L::KS>(kst, c, kbuf(0));
      store_chunk<L::KS>(pre, c, kbuf(1));
      store_chunk<L::VS>(vst, c, vbuf(0));
    }
    if constexpr (CHAIN) {
      load_stream(kst, false, kt_l, kt_t, kt_off);
      load_stream(vst, true, vt_l, vt_t, vt_off);
    } else {
      load_sub(kst, false, 2);
      load_sub(vst, true, 1);
    }
    __syncthreads();
    Scores sa, sb;
    POps pb;
    Ops ops;
#pragma unroll
    for (int j = 0; j < PF; ++j) ops[j] = kread(kbuf(0), j);
    // P carries both groups' staging of interval 0
    if (len() > 1) phase_a<true, false, 1, true>(st, sa, sa, pb, ops, kbuf(0), kbuf(1), 0);
    else phase_a<true, false, 2, true>(st, sa, sa, pb, ops, kbuf(0), vbuf(0), 0);
    max_all(st, sa, 0, tpos);
    if (!grp) __syncthreads();
    // two subtiles per iteration so that the score buffers keep their roles (S(i) in sa
    // for even i); the last ones move S(i+1) into sa instead
    int i = 0;
    for (; i + 3 < len(); i += 2) {
      iter<0>(st, sa, sb, pb, ops, i, tpos, next_q, bound);
      iter<0>(st, sb, sa, pb, ops, i + 1, tpos, next_q, bound);
    }
    if (i + 3 == len()) {
      iter<0>(st, sa, sb, pb, ops, i, tpos, next_q, bound);
      copy_scores(sa, sb);
      ++i;
    }
    if (i + 2 == len()) {
      iter<1>(st, sa, sb, pb, ops, i, tpos, next_q, bound);
      copy_scores(sa, sb);
      ++i;
    }
    iter<2>(st, sa, sb, pb, ops, i, tpos, next_q, bound);
    if (grp) __syncthreads();
  }
};

// The wave's rows over keys [key_begin, key_end) of one kv-head; subtiles whose last
// key exceeds diag_from (the smallest query position of the workgroup) or key_end are
// masked.  load_queries() fills st (query operands and the initial state); it runs
// after the walker's first K/V loads are issued.
template <int D, int QT, typename QueryLoad>
__device__ __forceinline__ void attend_range(WaveState<D, QT>& st, char* lds,
                                             const uint16_t* __restrict__ kbase,
                                             const uint16_t* __restrict__ vbase, size_t rs,
                                             int key_begin, int key_end, float sl,
                                             int diag_from, const int (&tpos)[QT],
                                             QueryLoad&& load_queries) {
  Walker<D, QT> w;
  w.lds = (lds_char*)lds;
  w.kbase = kbase;
  w.vbase = vbase;
  w.rs = rs;
  w.key_begin = key_begin;
  w.key_end = key_end;
  w.diag_from = diag_from;
  w.sl = sl;
  // waves w and w + kAttnWaves/2 share a SIMD (waves are dealt to SIMDs in turn), so
  // the halves of the workgroup are the two groups
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  w.grp = wave / (kAttnWaves / 2);
  w.begin();
  load_queries();
  w.run(st, tpos, [](int) {}, [](int) {});
}

// value held by lane (lane ^ 1): a DPP quad permute [1, 0, 3, 2]
__device__ __forceinline__ uint32_t swap_adjacent(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);
}

// normalise and store one query tile's partial: o rounded to bf16 (nearest even) [D],
// lse (natural log) in fp32.  Every lane of the wavefront must call it (with PAIRED
// the lanes exchange data); only valid rows are written.
//
// Lane (n, hf) holds dims dt*32 + ii*8 + hf*4 + r of its row, in 16-byte chunks
// c = (dt, ii / 2).  Chunk c of lane hf is stored at position c*16 + hf*8, next to
// the same chunk of the pair's other lane, so each store (and each merge load) moves
// 32 contiguous bytes of a row: half the memory requests of storing each lane's half
// row apart (at 64K tokens with 128-key blocks, history 4.85 -> 4.29 ms).
//
// PAIRED: a row's 64-byte segment s holds chunks 2s and 2s+1 of both lanes.  The
// lanes of rows n and n ^ 1 trade one chunk per segment, and each store then writes
// whole 64-byte segments: the lanes of row 2m write its chunk 2s and those of row 2m+1
// its chunk 2s+1 (first store), and the reverse for row 2m+1 (second store).  Half
// the requests again (64K with 128-key blocks: 4.24 -> 3.89 ms, same bytes); in the
// MFMA-bound chained kernel the exchange costs more than it saves (+0.4% at 128K).
template <int D, int QT, bool PAIRED = false>
__device__ __forceinline__ void store_partial(const WaveState<D, QT>& st, int qt, bool valid,
                                              uint16_t* __restrict__ po, float* __restrict__ pl) {
  const int lane = threadIdx.x & 63, hf = lane >> 5;
  const float ltot = pair_sum(st.l[qt]);
  if (!PAIRED && !valid) return;
  const float inv = 1.f / ltot;
  u32x4_t wc[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int i2 = 0; i2 < 2; ++i2) {
      const f32x16_t& o = st.o[qt][dt];
      const int a = 8 * i2;
      wc[dt * 2 + i2] = u32x4_t{pack_bf16x2(o[a] * inv, o[a + 1] * inv),
                                pack_bf16x2(o[a + 2] * inv, o[a + 3] * inv),
                                pack_bf16x2(o[a + 4] * inv, o[a + 5] * inv),
                                pack_bf16x2(o[a + 6] * inv, o[a + 7] * inv)};
    }
  if (PAIRED) {
    const bool odd = lane & 1;
    const uint64_t pa = reinterpret_cast<uint64_t>(po);
    const uint64_t pb = ((uint64_t)swap_adjacent((uint32_t)(pa >> 32)) << 32) |
                        swap_adjacent((uint32_t)pa);
    const bool pvalid = swap_adjacent(valid ? 1u : 0u) != 0u;
    char* const row_e = reinterpret_cast<char*>(odd ? pb : pa);
    char* const row_o = reinterpret_cast<char*>(odd ? pa : pb);
    const bool ve = odd ? pvalid : valid, vo = odd ? valid : pvalid;
    const int off = (odd ? 32 : 0) + 16 * hf;
#pragma unroll
    for (int sg = 0; sg < D / 32; ++sg) {
      const u32x4_t E = wc[2 * sg], O = wc[2 * sg + 1];
      u32x4_t x;
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = swap_adjacent(odd ? E[i] : O[i]);
      const u32x4_t a = odd ? x : E, b = odd ? O : x;
      if (ve) *reinterpret_cast<u32x4_t*>(row_e + 64 * sg + off) = a;
      if (vo) *reinterpret_cast<u32x4_t*>(row_o + 64 * sg + off) = b;
    }
    if (!valid) return;
  } else {
#pragma unroll
    for (int c = 0; c < D / 16; ++c)
      *reinterpret_cast<u32x4_t*>(po + c * 16 + hf * 8) = wc[c];
  }
  if (hf == 0) *pl = (st.m[qt] + __log2f(ltot)) * 0.69314718055994530942f;
}

// The parts are read CH at a time so that their loads are in flight together.
#ifndef MOBA_MERGE_CH
#define MOBA_MERGE_CH 4
#endif
constexpr int kMergeCH = MOBA_MERGE_CH;

// the lane's chunks of part rows s0 .. s0 + CH - 1 (see store_partial); indices past nh
// are clamped to the row's last part (their weight is 0)
template <int D, int CH>
struct PartRows {
  u32x4_t x[CH][D / 16];
};
template <int D, int CH>
__device__ __forceinline__ void load_parts(PartRows<D, CH>& p, const uint16_t* __restrict__ po,
                                           int s0, int nh, int hf) {
#pragma unroll
  for (int u = 0; u < CH; ++u) {
    const uint16_t* ps = po + (size_t)min(s0 + u, nh - 1) * D + hf * 8;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) p.x[u][c] = *reinterpret_cast<const u32x4_t*>(ps + c * 16);
  }
}
// acc += sum_u w[u] * part row u, parts in order
template <int D, int CH>
__device__ __forceinline__ void add_parts(f32x4_t (&acc)[D / 32][4], const PartRows<D, CH>& p,
                                          const float (&w)[CH]) {
#pragma unroll
  for (int u = 0; u < CH; ++u)
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const u32x4_t& xc = p.x[u][dt * 2 + ii / 2];
        const u32x2_t y = {xc[(ii & 1) * 2], xc[(ii & 1) * 2 + 1]};
        const float xf[4] = {__uint_as_float(y[0] << 16), __uint_as_float(y[0] & 0xffff0000u),
                             __uint_as_float(y[1] << 16), __uint_as_float(y[1] & 0xffff0000u)};
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[dt][ii][r] = fmaf(w[u], xf[r], acc[dt][ii][r]);
      }
}
template <int D>
__device__ __forceinline__ void store_merged(const f32x4_t (&acc)[D / 32][4], float L, int hf,
                                             uint16_t* __restrict__ orow,
                                             float* __restrict__ lrow) {
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      u32x2_t pk;
      pk[0] = f32_to_bf16_rne(acc[dt][ii][0]) | (f32_to_bf16_rne(acc[dt][ii][1]) << 16);
      pk[1] = f32_to_bf16_rne(acc[dt][ii][2]) | (f32_to_bf16_rne(acc[dt][ii][3]) << 16);
      *reinterpret_cast<u32x2_t*>(orow + dt * 32 + ii * 8 + hf * 4) = pk;
    }
  if (hf == 0) *lrow = L;
}

// Merge of a row with 1 <= nh <= NL parts: the NL lse values (clamped indices) and the
// first CHF part rows are loaded in one round, the lse then stay in registers, so the
// merge waits on ceil(nh / CHF) rounds of loads instead of re-reading the lse for the
// max, the sum and the weights.  Same arithmetic, in the same order, as the general
// path.  Two part rows per round: at 128K (11 parts) the current-block kernel takes
// 6.30 -> 6.12 ms, at 64K with 128-key blocks (15 parts) 2.30 -> 2.17 ms, bit for bit
// the same; rounds of three or four part rows spill (the walk's registers are not all
// free at the end).
#ifndef MOBA_MERGE_CHF
#define MOBA_MERGE_CHF 2
#endif
template <int D, int QT, int NL>
__device__ __forceinline__ void merge_store_regs(const WaveState<D, QT>& st, int qt, int nh,
                                                 float lc, float lse_c,
                                                 const uint16_t* __restrict__ po,
                                                 const float* __restrict__ pl, size_t ls,
                                                 int hf, uint16_t* __restrict__ orow,
                                                 float* __restrict__ lrow) {
  constexpr int CH = MOBA_MERGE_CHF;
  float lv[NL];
#pragma unroll
  for (int u = 0; u < NL; ++u) lv[u] = pl[(size_t)min(u, nh - 1) * ls];
  PartRows<D, CH> p;
  load_parts<D, CH>(p, po, 0, nh, hf);
  float mx = lse_c;
#pragma unroll
  for (int u = 0; u < NL; ++u) mx = fmaxf(mx, lv[u]);
  float den = expf(lse_c - mx);
#pragma unroll
  for (int u = 0; u < NL; ++u)
    if (u < nh) den += expf(lv[u] - mx);
  const float L = mx + logf(den);
  const float wc = expf(lse_c - L) / lc;
  f32x4_t acc[D / 32][4];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[dt][ii][r] = st.o[qt][dt][ii * 4 + r] * wc;
#pragma unroll
  for (int s0 = 0; s0 < NL; s0 += CH) {
    if (s0 >= nh) break;
    if (s0 > 0) load_parts<D, CH>(p, po, s0, nh, hf);
    float w[CH];
#pragma unroll
    for (int u = 0; u < CH; ++u)
      w[u] = (s0 + u < NL && s0 + u < nh) ? expf(lv[s0 + u < NL ? s0 + u : 0] - L) : 0.f;
    add_parts<D, CH>(acc, p, w);
  }
  store_merged<D>(acc, L, hf, orow, lrow);
}

// Log-sum-exp merge of a row's current-block result (in registers) with its nh history
// partials, written as the final output: L = ln(e^lse_c + sum_s e^lse_s), out =
// e^(lse_c - L) o_c + sum_s e^(lse_s - L) o_s (bf16, round to nearest even), lse = L.
// Lane (n, hf) holds dims dt*32 + ii*8 + hf*4 + r of its row; the row's part lse of
// slot s is pl[s * ls].
template <int D, int QT>
__device__ __forceinline__ void merge_store(const WaveState<D, QT>& st, int qt, bool valid,
                                            int nh, const uint16_t* __restrict__ po,
                                            const float* __restrict__ pl, size_t ls,
                                            uint16_t* __restrict__ orow, float* __restrict__ lrow) {
  const int lane = threadIdx.x & 63, hf = lane >> 5;
  const float lc = pair_sum(st.l[qt]);
  if (!valid) return;
  const float ln2 = 0.69314718055994530942f;
  const float lse_c = (st.m[qt] + __log2f(lc)) * ln2;
  // nh is the same for every row of a workgroup (min(block, k - 1))
  if (nh >= 1 && nh <= 4)
    return merge_store_regs<D, QT, 4>(st, qt, nh, lc, lse_c, po, pl, ls, hf, orow, lrow);
  if (nh >= 1 && nh <= 8)
    return merge_store_regs<D, QT, 8>(st, qt, nh, lc, lse_c, po, pl, ls, hf, orow, lrow);
  if (nh >= 1 && nh <= 16)
    return merge_store_regs<D, QT, 16>(st, qt, nh, lc, lse_c, po, pl, ls, hf, orow, lrow);
  // general path (no parts, or more than 16): the lse are read again for each use
  constexpr int CH = kMergeCH;
  float mx = lse_c;
  for (int s0 = 0; s0 < nh; s0 += CH) {
    float v[CH];
#pragma unroll
    for (int u = 0; u < CH; ++u) v[u] = pl[(size_t)min(s0 + u, nh - 1) * ls];
#pragma unroll
    for (int u = 0; u < CH; ++u) mx = fmaxf(mx, v[u]);
  }
  float den = expf(lse_c - mx);
  for (int s0 = 0; s0 < nh; s0 += CH) {
    float v[CH];
#pragma unroll
    for (int u = 0; u < CH; ++u) v[u] = pl[(size_t)min(s0 + u, nh - 1) * ls];
#pragma unroll
    for (int u = 0; u < CH; ++u)
      if (s0 + u < nh) den += expf(v[u] - mx);
  }
  const float L = mx + logf(den);
  const float wc = expf(lse_c - L) / lc;
  f32x4_t acc[D / 32][4];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[dt][ii][r] = st.o[qt][dt][ii * 4 + r] * wc;
  for (int s0 = 0; s0 < nh; s0 += CH) {
    PartRows<D, CH> p;
    load_parts<D, CH>(p, po, s0, nh, hf);
    float w[CH];
#pragma unroll
    for (int u = 0; u < CH; ++u)
      w[u] = s0 + u < nh ? expf(pl[(size_t)min(s0 + u, nh - 1) * ls] - L) : 0.f;
    add_parts<D, CH>(acc, p, w);
  }
  store_merged<D>(acc, L, hf, orow, lrow);
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
// One workgroup = one tile of up to kAttnWaves * 32 * QT gathered rows of one list
// (b, g, j).
template <int D, int QT>
__global__ __launch_bounds__(kAttnThreads, MOBA_ATTN_WPE) void attn_history_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, SeqMap sq, int hq, int hkv, int block, int topk,
    float sl, int g0, int ng, int nb, const int4* __restrict__ tiles,
    const int32_t* __restrict__ tile_count, const uint32_t* __restrict__ entries,
    uint16_t* __restrict__ part_o, float* __restrict__ part_lse, size_t ls) {
  __shared__ __attribute__((aligned(16))) char lds[Lds<D>::TOTAL];
  const int tile_id = blockIdx.x;
  if (tile_id >= *tile_count) return;
  const int4 tl = tiles[tile_id];
  const int list = tl.x;
  const int j = list % nb, gi = (list / nb) % ng, b = list / (nb * ng);
  const int tok0 = sq.tok0(b);
  const int G = hq / hkv, g = g0 + gi;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, n = lane & 31;

  WaveState<D, QT> st;
  int tq[QT], hlq[QT], slq[QT], tpos[QT];
  bool vq[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) tpos[qt] = 0x7fffffff;    // history keys all precede
  const size_t rs = (size_t)hkv * D;
  const uint16_t* kbase = k + ((size_t)tok0 * hkv + g) * D;
  const uint16_t* vbase = v + ((size_t)tok0 * hkv + g) * D;
  const int key_begin = j * block;
  attend_range<D, QT>(st, lds, kbase, vbase, rs, key_begin, key_begin + block, sl,
                      0x7fffffff, tpos, [&] {
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const int e = tl.y + (wave * QT + qt) * 32 + n;
      vq[qt] = e < tl.z;
      const uint32_t ent = vq[qt] ? entries[e] : 0u;
      const int sb = entry_slot_bits(topk);
      slq[qt] = (int)(ent & ((1u << sb) - 1u));
      const int rr = (int)(ent >> sb);
      tq[qt] = rr / G;
      hlq[qt] = rr % G;
      const uint16_t* qrow = q + ((size_t)((size_t)tok0 + tq[qt]) * hq + g * G + hlq[qt]) * D;
      load_q(st, qt, qrow, vq[qt]);
    }
    state_init(st);
  });
  const int ngq = ng * G;
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const size_t row = sq.prow(b, gi * G + hlq[qt], ngq) + tq[qt];
    store_partial(st, qt, vq[qt], part_o + (row * (topk - 1) + slq[qt]) * D,
                  part_lse + (size_t)slq[qt] * ls + row);
  }
}

// ------------------------------------------------------ history, persistent (a4)
// The same attention as attn_history_kernel, but one workgroup per CU walks all of its
// tiles (its first, tile blockIdx.x, then those it takes from the tile queue) as one
// continuous walk: the
// staging runs into the next tile's block while the current tile finishes, the next
// tile's query rows load during the last PV phase of the current one, and its first
// QK^T shares a phase with the current tile's last exponentials.  So a tile pays no
// prologue (first K/V loads, query gather, pipeline fill) and no workgroup launch, which
// in the one-tile-per-workgroup kernel are a fixed cost of a few microseconds per tile.
template <int D>
__global__ __launch_bounds__(kAttnThreads, MOBA_ATTN_WPE) void attn_history_chain_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, SeqMap sq, int hq, int hkv, int block, int topk,
    float sl, int g0, int ng, int nb, const int4* __restrict__ tiles,
    int32_t* __restrict__ tile_count, const uint32_t* __restrict__ entries,
    uint16_t* __restrict__ part_o, float* __restrict__ part_lse, size_t ls) {
  __shared__ __attribute__((aligned(16))) char lds[Lds<D>::TOTAL];
  __shared__ int tq[4];
  const int ntiles = *tile_count;
  if ((int)blockIdx.x >= ntiles) return;
  // Tiles 0 .. gridDim.x - 1 go to the workgroups in order, the rest through the queue
  // counter after the tile count (zero at launch): a workgroup that finishes its tiles
  // early takes more, so the CUs finish together however their speeds differ.
  int32_t* queue = tile_count + 1;
  if (threadIdx.x == 0) {
    tq[0] = blockIdx.x;
    tq[1] = (int)gridDim.x + atomicAdd(queue, 1);
  }
  __syncthreads();
  const int G = hq / hkv, ngq = ng * G;
  const int wave = threadIdx.x >> 6, n = threadIdx.x & 31;
  const int sb = entry_slot_bits(topk);
  Walker<D, 1, true> w;
  w.tq = (__attribute__((address_space(3))) int*)tq;
  w.ntiles = ntiles;
  w.ntw = __builtin_amdgcn_readfirstlane(tq[1]) < ntiles ? ntiles : 1;
  w.queue = queue;
  // this lane's index entry in the workgroup's tile s (all ones: no row)
  auto entry_of = [&](int s) -> uint32_t {
    const int4 tl = tiles[w.tile_of(s)];
    const int e = tl.y + wave * 32 + n;
    return e < tl.z ? entries[e] : 0xffffffffu;
  };
  auto tile_bg = [&](int s, int& b, int& gi) {
    const int list = tiles[w.tile_of(s)].x;
    gi = (list / nb) % ng;
    b = list / (nb * ng);
  };
  WaveState<D, 1> st;
  const int tpos[1] = {0x7fffffff};    // history keys all precede the rows
  auto load_tile_q = [&](int s, uint32_t ent) {
    int b, gi;
    tile_bg(s, b, gi);
    const bool valid = ent != 0xffffffffu;
    const int rr = valid ? (int)(ent >> sb) : 0;
    load_q(st, 0, q + ((size_t)((size_t)sq.tok0(b) + rr / G) * hq + (g0 + gi) * G + rr % G) * D,
           valid);
  };
  auto store_tile = [&](int s, uint32_t ent) {
    int b, gi;
    tile_bg(s, b, gi);
    const bool valid = ent != 0xffffffffu;
    const int rr = valid ? (int)(ent >> sb) : 0;
    const int slot = (int)(ent & ((1u << sb) - 1u));
    const size_t row = sq.prow(b, gi * G + rr % G, ngq) + rr / G;
    store_partial(st, 0, valid, part_o + (row * (topk - 1) + slot) * D,
                  part_lse + (size_t)slot * ls + row);
  };
  w.lds = (lds_char*)lds;
  w.kbase = k;
  w.vbase = v;
  w.rs = (size_t)hkv * D;
  w.key_begin = 0;
  w.key_end = block;
  w.diag_from = 0x7fffffff;
  w.sl = sl;
  w.grp = __builtin_amdgcn_readfirstlane(wave) / (kAttnWaves / 2);
  w.tiles = tiles;
  w.nb = nb;
  w.ng = ng;
  w.g0 = g0;
  w.hkv = hkv;
  w.sq = sq;
  w.begin();
  uint32_t ent_cur = entry_of(0);
  uint32_t ent_nx = w.ntw > 1 ? entry_of(1) : 0xffffffffu;
  load_tile_q(0, ent_cur);
  state_init(st);
  w.run(st, tpos, [&](int s) { load_tile_q(s, ent_nx); },
        [&](int s) {
          store_tile(s, ent_cur);
          state_init(st);
          ent_cur = ent_nx;
          ent_nx = s + 2 < w.ntw ? entry_of(s + 2) : 0xffffffffu;
        });
  store_tile(w.ntw - 1, ent_cur);
  // the last tile's queue request may still be in flight (its answer is not needed)
  __builtin_amdgcn_s_waitcnt(0);
}

// ------------------------------------------------- history, blocks of <= 128 keys (a4)
// For small blocks (FlashMoBA story, paragraph on running many small blocks: short
// tiles, scattered access and task granularity) the whole block, K and V, fits in LDS
// (75.8 KB at 128 keys and d = 128, so two workgroups share a CU).  A workgroup of
// four waves stages its block once and then streams the block's gathered query rows
// through it: each wave takes 32-row groups in turn and, for each, computes the scores
// of all NH*32 keys, the exact row max, the exponentials, P V and the normalised
// partial.  After the staging there is no barrier, so the two waves of a SIMD (from
// the two workgroups) drift out of phase and overlap one's exponentials with the
// other's MFMAs; the next group's entries and query rows are loaded ahead.  A tile of
// the index holds up to kResidentTileRows rows, 8x the streaming kernel's, so a block
// is staged once per 2048 rows instead of once per 256.  Keys past the block's end (a
// block of 16, 48, ... keys) are masked and read zero rows.
constexpr int kResidentWaves = 4;
constexpr int kResidentTileRows = 2048;

template <int D, int NH>
struct ResidentLds {
  using L = Lds<D>;
  static constexpr int KEYS = 32 * NH;
  static constexpr int KBYTES = KEYS * L::KS;
  static constexpr int TOTAL = KEYS * (L::KS + L::VS);
};

template <int D, int NH>
__global__ __launch_bounds__(64 * kResidentWaves, 2) void attn_history_resident_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, SeqMap sq, int hq, int hkv, int block, int topk,
    float sl, int g0, int ng, int nb, const int4* __restrict__ tiles,
    const int32_t* __restrict__ tile_count, const uint32_t* __restrict__ entries,
    uint16_t* __restrict__ part_o, float* __restrict__ part_lse, size_t ls) {
  using L = Lds<D>;
  using RL = ResidentLds<D, NH>;
  constexpr int KS = D / 16;                  // MFMA k-steps over the head dim
  constexpr int NPK = 2 * NH;                 // 16-key k-steps of P V
  __shared__ __attribute__((aligned(16))) char lds[RL::TOTAL];
  char* kl = lds;
  char* vl = lds + RL::KBYTES;
  const int tile_id = blockIdx.x;
  if (tile_id >= *tile_count) return;
  const int4 tl = tiles[tile_id];
  const int list = tl.x;
  const int j = list % nb, gi = (list / nb) % ng, b = list / (nb * ng);
  const int tok0 = sq.tok0(b);
  const int G = hq / hkv, g = g0 + gi;
  const size_t rs = (size_t)hkv * D;
  const int key0 = j * block;
  const int nkeys = min(block, sq.len(b) - key0);   // a history block is whole; be safe

  // stage K and V of the block into padded LDS rows; rows past nkeys are zero
  {
    constexpr int CPR = D / 8;
    for (int c = threadIdx.x; c < RL::KEYS * CPR; c += 64 * kResidentWaves) {
      const int row = c / CPR, col = c % CPR;
      u32x4_t kx = {0u, 0u, 0u, 0u}, vx = {0u, 0u, 0u, 0u};
      if (row < nkeys) {
        const size_t off = ((size_t)tok0 + key0 + row) * rs + (size_t)g * D + col * 8;
        kx = *reinterpret_cast<const u32x4_t*>(k + off);
        vx = *reinterpret_cast<const u32x4_t*>(v + off);
      }
      *reinterpret_cast<u32x4_t*>(kl + row * L::KS + col * 16) = kx;
      *reinterpret_cast<u32x4_t*>(vl + row * L::VS + col * 16) = vx;
    }
  }
  __syncthreads();

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, n = lane & 31, hf = lane >> 5;
  const int ngq = ng * G;
  const int sb = entry_slot_bits(topk);
  const int ngroups = (tl.z - tl.y + 31) / 32;
  const char* kp = kl + n * L::KS + hf * 16;
  const char* vp = vl + (4 * hf + ((lane & 15) >> 2)) * L::VS +
                   (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;

  // entry of this lane's row in group rg, and that row's query operands.  The loads
  // are paired like the partial stores: each load instruction reads whole 64-byte
  // segments (chunks 2s and 2s+1 of both lanes of a row), the lanes of rows n and
  // n ^ 1 loading for each other, and pair_qops trades the chunks before the QK
  // MFMAs (64K with 128-key blocks: 3.91 -> 3.85 ms, bit-identical).
  auto entry_of = [&](int rg) -> uint32_t {
    const int e = tl.y + rg * 32 + n;
    return (rg < ngroups && e < tl.z) ? entries[e] : 0xffffffffu;
  };
  auto load_qops = [&](uint32_t ent, bf16x8_t (&bq)[KS]) {
    const bool valid = ent != 0xffffffffu;
    const int rr = valid ? (int)(ent >> sb) : 0;
    const uint16_t* qrow = q + ((size_t)((size_t)tok0 + rr / G) * hq + g * G + rr % G) * D;
    const bool odd = lane & 1;
    const uint64_t pa = reinterpret_cast<uint64_t>(qrow);
    const uint64_t pb = ((uint64_t)swap_adjacent((uint32_t)(pa >> 32)) << 32) |
                        swap_adjacent((uint32_t)pa);
    const bool pvalid = swap_adjacent(valid ? 1u : 0u) != 0u;
    const char* const row_e = reinterpret_cast<const char*>(odd ? pb : pa);
    const char* const row_o = reinterpret_cast<const char*>(odd ? pa : pb);
    const bool ve = odd ? pvalid : valid, vo = odd ? valid : pvalid;
    const int off = (odd ? 32 : 0) + 16 * hf;
#pragma unroll
    for (int sg = 0; sg < KS / 2; ++sg) {
      u32x4_t a = {0u, 0u, 0u, 0u}, bb = {0u, 0u, 0u, 0u};
      if (ve) a = *reinterpret_cast<const u32x4_t*>(row_e + 64 * sg + off);
      if (vo) bb = *reinterpret_cast<const u32x4_t*>(row_o + 64 * sg + off);
      bq[2 * sg] = as_bf16x8(a);
      bq[2 * sg + 1] = as_bf16x8(bb);
    }
  };
  // after load_qops, before the operands are used: the pair's lanes trade the chunks
  // they loaded for each other
  auto pair_qops = [&](bf16x8_t (&bq)[KS]) {
    const bool odd = lane & 1;
#pragma unroll
    for (int sg = 0; sg < KS / 2; ++sg) {
      const u32x4_t a = __builtin_bit_cast(u32x4_t, bq[2 * sg]);
      const u32x4_t bb = __builtin_bit_cast(u32x4_t, bq[2 * sg + 1]);
      u32x4_t x;
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = swap_adjacent(odd ? a[i] : bb[i]);
      bq[2 * sg] = as_bf16x8(odd ? x : a);
      bq[2 * sg + 1] = as_bf16x8(odd ? bb : x);
    }
  };

  // One 32-row group with query operands bq: scores, softmax, P V, partial store.
  // `refill` runs right after the QK MFMAs, when bq is free: it loads a later group's
  // query rows into bq.
  auto group = [&](int rg, uint32_t ent_cur, bf16x8_t (&bq)[KS], auto&& refill) {
    pair_qops(bq);
    // scores S^T = K Q^T over every key of the block
    f32x16_t sc[NH];
#pragma unroll
    for (int kk = 0; kk < NH; ++kk)
#pragma unroll
      for (int i = 0; i < 16; ++i) sc[kk][i] = 0.f;
    {
      // MFMA j takes k-step j / NH of key half j % NH (the NH accumulators alternate);
      // the K operand reads run PF ahead
      constexpr int NQ = KS * NH, PF = 4;
      auto kread = [&](int jj) {
        return as_bf16x8(*reinterpret_cast<const u32x4_t*>(kp + (jj % NH) * 32 * L::KS +
                                                            (jj / NH) * 32));
      };
      bf16x8_t ka[NQ];
#pragma unroll
      for (int jj = 0; jj < PF && jj < NQ; ++jj) ka[jj] = kread(jj);
#pragma unroll
      for (int jj = 0; jj < NQ; ++jj) {
        if (jj + PF < NQ) ka[jj + PF] = kread(jj + PF);
        sc[jj % NH] = mfma32x32x16(ka[jj], bq[jj / NH], sc[jj % NH]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    refill();
    // keys past the block's end
    if (nkeys < RL::KEYS) {
#pragma unroll
      for (int kk = 0; kk < NH; ++kk)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (kk * 32 + (e >> 2) * 8 + hf * 4 + (e & 3) >= nkeys) sc[kk][e] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kk = 0; kk < NH; ++kk)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sc[kk][e]);
    const float m = pair_max(mx) * sl;
    // exponentials 16 keys at a time, each slice packed and taken by its P V MFMAs at
    // once (O^T = V^T P^T), so only one slice of P is ever held
    float rsum = 0.f;
    WaveState<D, 1> st;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) st.o[0][dt][i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < NPK; ++ks) {
      // the slice's V^T operands first: its exponentials cover their LDS latency
      u32x4_t va[D / 32];
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        const u32x2_t lo = lds_read_tr16(vp + (16 * ks) * L::VS + dt * 64);
        const u32x2_t hi = lds_read_tr16(vp + (16 * ks + 8) * L::VS + dt * 64);
        va[dt] = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
      }
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int x = 8 * ks + e;
        p[e] = __builtin_amdgcn_exp2f(fmaf(sc[x >> 4][x & 15], sl, -m));
        rsum += p[e];
      }
      const bf16x8_t pb = as_bf16x8(u32x4_t{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                                            pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])});
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
        st.o[0][dt] = mfma32x32x16(as_bf16x8(va[dt]), pb, st.o[0][dt]);
      __builtin_amdgcn_sched_barrier(0);
    }
    st.m[0] = m;
    st.l[0] = rsum;
    const bool valid = ent_cur != 0xffffffffu;
    const int rr = valid ? (int)(ent_cur >> sb) : 0;
    const int slot = (int)(ent_cur & ((1u << sb) - 1u));
    const size_t row = sq.prow(b, gi * G + rr % G, ngq) + rr / G;
    store_partial<D, 1, true>(st, 0, valid, part_o + (row * (topk - 1) + slot) * D,
                              part_lse + (size_t)slot * ls + row);
  };

  constexpr int W = kResidentWaves;
  // Groups in pairs, two buffers of query operands: group rg computes on qa while qb
  // holds group rg + W; after rg's QK, qa takes group rg + 2W.  Entries run four
  // groups ahead, so neither the entry nor the query rows it names is waited for in
  // the group that needs them.
  uint32_t e0 = entry_of(wave), e1 = entry_of(wave + W);
  uint32_t e2 = entry_of(wave + 2 * W), e3 = entry_of(wave + 3 * W);
  bf16x8_t qa[KS], qb[KS];
  load_qops(e0, qa);
  load_qops(e1, qb);
  for (int rg = wave; rg < ngroups; rg += 2 * W) {
    const uint32_t c0 = e0, c1 = e1;
    e0 = e2;
    e1 = e3;
    e2 = entry_of(rg + 4 * W);
    e3 = entry_of(rg + 5 * W);
    group(rg, c0, qa, [&] { load_qops(e0, qa); });
    if (rg + W >= ngroups) break;
    group(rg + W, c1, qb, [&] { load_qops(e1, qb); });
  }
}

// ---------------------------------------------------------------- current (a5)
// One workgroup = a run of consecutive tokens of block c for the query heads of
// kv-head g; all its waves share every staged K/V subtile.  With G heads per kv-head
// dividing the wave count, wave w takes head w % G and 32*QT-token sub-tile w / G;
// otherwise one sub-tile and the heads in rounds.  Tiles run from the end of the
// block backwards, so the longest ones start first.
//
// The dispatcher deals workgroup L (x fastest, then y, then z) to XCD L % 8, and each
// XCD has its own L2.  When the number of (block, head group) lists is a multiple of
// 8, the linear id is remapped so that every XCD takes whole lists: the 64 workgroups
// that stage one block's K/V then share one L2 instead of fetching it into all eight
// (11% faster at 128K with B = 4096).
__host__ __device__ __forceinline__ int current_subtiles(int G) {
  return (G <= kAttnWaves && kAttnWaves % G == 0) ? kAttnWaves / G : 1;
}

template <int D, int QT>
__global__ __launch_bounds__(kAttnThreads, MOBA_ATTN_WPE) void attn_current_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, SeqMap sq, int hq, int hkv, int block, int topk,
    float sl, int g0, int ng, const uint16_t* __restrict__ part_o,
    const float* __restrict__ part_lse, size_t ls, uint16_t* __restrict__ out,
    float* __restrict__ lse) {
  __shared__ __attribute__((aligned(16))) char lds[Lds<D>::TOTAL];
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
  const int gi = bz % ng, b = bz / ng;
  const int G = hq / hkv, g = g0 + gi;
  const int TS = current_subtiles(G);
  const int TT = 32 * QT * TS;
  const int x = gridDim.x - 1 - bx;
  const int t0 = c * block + x * TT;
  const int Tb = sq.len(b), tok0 = sq.tok0(b);
  // a partial last block, or a block past the end of a shorter packed sequence
  const int t_end = min(min(t0 + TT, (c + 1) * block), Tb);
  if (t0 >= t_end) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, n = lane & 31;
  const int hw = TS > 1 ? wave % G : wave;      // head of this wave within a round
  const int tsub = TS > 1 ? wave / G : 0;
  const int hstep = TS > 1 ? G : kAttnWaves;     // heads covered per round
  const size_t rs = (size_t)hkv * D;
  const uint16_t* kbase = k + ((size_t)tok0 * hkv + g) * D;
  const uint16_t* vbase = v + ((size_t)tok0 * hkv + g) * D;
  const int ngq = ng * G;
  for (int round = 0; round * hstep < G; ++round) {
    const int hl = round * hstep + hw;
    const bool active = hl < G;
    WaveState<D, QT> st;
    int tpos[QT];
    bool vq[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      tpos[qt] = t0 + (tsub * QT + qt) * 32 + n;
      vq[qt] = active && tpos[qt] < t_end;
    }
    // waves without a head this round run on zero queries: every wave takes part in
    // every phase and barrier of the walker
    attend_range<D, QT>(st, lds, kbase, vbase, rs, c * block, t_end, sl, t0, tpos, [&] {
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        const uint16_t* qrow = q + ((size_t)((size_t)tok0 + (vq[qt] ? tpos[qt] : 0)) * hq +
                                    g * G + (active ? hl : 0)) * D;
        load_q(st, qt, qrow, vq[qt]);
      }
      state_init(st);
    });
    if (active) {
      const int nh = min(c, topk - 1);   // history slots of every row of this block
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        const int t = vq[qt] ? tpos[qt] : 0;
        const size_t row = sq.prow(b, gi * G + hl, ngq) + t;
        merge_store(st, qt, vq[qt], nh, part_o + row * (topk - 1) * D, part_lse + row, ls,
                    out + ((size_t)((size_t)tok0 + t) * hq + g * G + hl) * D,
                    lse + sq.lrow(b, g * G + hl, hq) + t);
      }
    }
  }
}

// ---------------------------------------------------------------- launchers
constexpr int kQT = MOBA_ATTN_QT;
int history_tile_rows() { return kAttnWaves * 32 * kQT; }
// Blocks of at most 128 keys run the resident kernel.  Its tiles are as long as
// kResidentTileRows while the launch still has >= 1024 of them (four per CU slot of
// its two workgroups per CU), and shorter, down to 128 rows, for small problems.
static bool history_resident(const Shape& s) { return s.block <= 128; }
int history_tile_rows(const Shape& s, long long n_entries) {
  if (!history_resident(s)) return history_tile_rows();
  int tm = kResidentTileRows;
  while (tm > 128 && n_entries / tm < 1024) tm /= 2;
  return tm;
}

// History partials of one pass (ng kv-heads): o is [row][slot][d] and lse [slot][row],
// rows as SeqMap::prow numbers them.  The lse of one slot are contiguous over rows, so
// the 32 rows of a wavefront (mostly consecutive tokens with the same slot) write and
// read whole 32-byte runs instead of one 4-byte word per (k-1)-float row.
static size_t part_lse_slot_stride(const Shape& s, int ng) {
  return s.cu ? (size_t)ng * s.G() * s.total : (size_t)s.b * ng * s.G() * s.T;
}

hipError_t launch_attn_history(const Shape& s, const uint16_t* q, const uint16_t* k,
                               const uint16_t* v, float scale, int g0, int ng,
                               const int4* tiles, int32_t* tile_count,
                               int max_tiles, const uint32_t* entries, uint16_t* part_o,
                               float* part_lse, hipStream_t st) {
  if (max_tiles <= 0) return hipSuccess;
  const float sl = scale * 1.4426950408889634f;
  if (history_resident(s)) {
    const int nh = (s.block + 31) / 32;
#define MOBA_RES(DD, NN)                                                                     \
  hipLaunchKernelGGL((attn_history_resident_kernel<DD, NN>), dim3(max_tiles),                  \
                     dim3(64 * kResidentWaves), 0, st, q, k, v, s.seqs(), s.hq, s.hkv, s.block, \
                     s.topk, sl, g0, ng, s.nb(), tiles, tile_count, entries, part_o, part_lse, \
                     part_lse_slot_stride(s, ng))
#define MOBA_RES_D(DD)            \
  do {                            \
    if (nh == 1) MOBA_RES(DD, 1); \
    else if (nh == 2) MOBA_RES(DD, 2); \
    else if (nh == 3) MOBA_RES(DD, 3); \
    else MOBA_RES(DD, 4);         \
  } while (0)
    if (s.d == 128) MOBA_RES_D(128);
    else MOBA_RES_D(64);
#undef MOBA_RES_D
#undef MOBA_RES
    return hipGetLastError();
  }
  // Blocks of 256 to 4096 keys run the persistent chained kernel, its workgroups taking
  // tiles from a queue.  Where a tile's fixed cost is a large share (32K tokens, B = 512:
  // walks of 8 subtiles) history takes 0.78 -> 0.74 ms; at 128K with B = 4096 it is
  // 0.3% faster than one tile per workgroup (67.5 -> 67.3 ms), bit for bit the same.
  // With a fixed round-robin assignment instead of the queue it was 2.4% slower there
  // (the CUs do not all run at the same speed).  The queue needs tiles of at least four
  // subtiles: the K staging stream, four subtiles ahead of the walk, enters tile it + 2
  // at subtile 2 * nsub - 5 of tile it, which must not come before subtile 2, where
  // every wave has read that tile's index.
#ifndef MOBA_CHAIN_MAXSUB
#define MOBA_CHAIN_MAXSUB 64
#endif
  if (s.block % KN == 0 && s.block >= 4 * KN && s.block <= MOBA_CHAIN_MAXSUB * KN &&
      (long long)max_tiles * (s.block / KN) < (1ll << 30)) {
    // one persistent workgroup per CU (the kernel's LDS allows one)
    int dev = 0, ncu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return hipErrorInvalidDevice;
    const int grid = std::max(1, std::min(max_tiles, ncu));
    if (s.d == 128)
      hipLaunchKernelGGL((attn_history_chain_kernel<128>), dim3(grid), dim3(kAttnThreads), 0, st,
                         q, k, v, s.seqs(), s.hq, s.hkv, s.block, s.topk, sl, g0, ng, s.nb(),
                         tiles, tile_count, entries, part_o, part_lse,
                         part_lse_slot_stride(s, ng));
    else
      hipLaunchKernelGGL((attn_history_chain_kernel<64>), dim3(grid), dim3(kAttnThreads), 0, st,
                         q, k, v, s.seqs(), s.hq, s.hkv, s.block, s.topk, sl, g0, ng, s.nb(),
                         tiles, tile_count, entries, part_o, part_lse,
                         part_lse_slot_stride(s, ng));
    return hipGetLastError();
  }
  if (s.d == 128)
    hipLaunchKernelGGL((attn_history_kernel<128, kQT>), dim3(max_tiles), dim3(kAttnThreads), 0,
                       st, q, k, v, s.seqs(), s.hq, s.hkv, s.block, s.topk, sl, g0, ng,
                       s.nb(), tiles, tile_count, entries, part_o, part_lse,
                       part_lse_slot_stride(s, ng));
  else
    hipLaunchKernelGGL((attn_history_kernel<64, kQT>), dim3(max_tiles), dim3(kAttnThreads), 0,
                       st, q, k, v, s.seqs(), s.hq, s.hkv, s.block, s.topk, sl, g0, ng,
                       s.nb(), tiles, tile_count, entries, part_o, part_lse,
                       part_lse_slot_stride(s, ng));
  return hipGetLastError();
}

hipError_t launch_attn_current(const Shape& s, const uint16_t* q, const uint16_t* k,
                               const uint16_t* v, float scale, int g0, int ng,
                               const uint16_t* part_o, const float* part_lse, uint16_t* out,
                               float* lse, hipStream_t st) {
  const float sl = scale * 1.4426950408889634f;
  const int TT = 32 * kQT * current_subtiles(s.G());
  dim3 grid((s.block + TT - 1) / TT, s.nb(), s.b * ng);
  if (s.d == 128)
    hipLaunchKernelGGL((attn_current_kernel<128, kQT>), grid, dim3(kAttnThreads), 0, st, q, k,
                       v, s.seqs(), s.hq, s.hkv, s.block, s.topk, sl, g0, ng, part_o,
                       part_lse, part_lse_slot_stride(s, ng), out, lse);
  else
    hipLaunchKernelGGL((attn_current_kernel<64, kQT>), grid, dim3(kAttnThreads), 0, st, q, k,
                       v, s.seqs(), s.hq, s.hkv, s.block, s.topk, sl, g0, ng, part_o,
                       part_lse, part_lse_slot_stride(s, ng), out, lse);
  return hipGetLastError();
}

}  // namespace moba
