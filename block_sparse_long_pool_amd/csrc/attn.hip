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
  static constexpr int TOTAL = 2 * (KBYTES + VBYTES);  // two K and two V buffers
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

// rows as they are, into padded LDS rows of STRIDE bytes
template <int D, int STRIDE>
__device__ __forceinline__ void tile_store(const TileRegs<D>& r, char* dst) {
  using R = TileRegs<D>;
  constexpr bool kAllThreads = (KN * R::CPR) % kAttnThreads == 0;
#pragma unroll
  for (int i = 0; i < R::NC; ++i) {
    const int ci = threadIdx.x + i * kAttnThreads;
    if (kAllThreads || ci < KN * R::CPR)
      *reinterpret_cast<u32x4_t*>(dst + (ci / R::CPR) * STRIDE + (ci % R::CPR) * 16) = r.c[i];
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

// Key-range walker, two wave groups in ping-pong.  The workgroup's waves form two
// groups (the two waves that share a SIMD are in different groups).  Every wave runs
// the same sequence of phases, separated by barriers:
//   P      QK^T of subtile 0, its mask and row max;
//   A(i)   the MFMAs of QK^T for subtile i+1 next to the exp/sum/pack of subtile i;
//   B(i)   the PV MFMAs of subtile i next to the mask and row max of subtile i+1,
//          then the lazy-rescale decision for subtile i+1;
// but group 1 starts one barrier later, so at every half-step h one wave of a SIMD is
// in an exp-heavy A phase while the other is in an MFMA/LDS-heavy phase.  Phase
// number f = 0 (P), 2i+1 (A(i)), 2i+2 (B(i)) runs at half-step h = f + group.
// LDS holds two K and two V buffers.  At half-step h all threads stage one slice
// each of one subtile, K(h/2 + 1) for even h and V(h/2) for odd h, from registers
// loaded two half-steps before.  K(j) is read at half-steps 2j-1 and 2j (K(0) at 0
// and 1) and V(i) at 2i+2 and 2i+3, so every buffer is rewritten only after both
// groups are done with its previous subtile.  Staging past the last subtile
// re-stages the last subtile into a buffer nobody reads again.
template <int D, int QT>
struct Walker {
  using L = Lds<D>;
  static constexpr int KSTEPS = D / 16;            // MFMA k-steps over the head dim
  static constexpr int NQK = NH * KSTEPS;          // QK^T MFMAs per query tile
  static constexpr int NPV = (KN / 16) * (D / 32); // PV MFMAs per query tile
#ifndef MOBA_ATTN_PFK
#define MOBA_ATTN_PFK 3
#endif
#ifndef MOBA_ATTN_PFV
#define MOBA_ATTN_PFV 4
#endif
  static constexpr int PFK = MOBA_ATTN_PFK, PFV = MOBA_ATTN_PFV;  // operand reads in flight
  static constexpr int NC = TileRegs<D>::NC;
  using Scores = f32x16_t[NH][QT];
  using POps = bf16x8_t[QT][KN / 16];
  char* lds;
  const uint16_t* kbase;
  const uint16_t* vbase;
  size_t rs;
  int key_begin, key_end, nsub, diag_from;
  float sl;
  int grp;                     // 0 leads, 1 trails by one half-step
  TileOffsets<D> to;
  TileRegs<D> bank[2];         // staging registers of even / odd phases

  __device__ __forceinline__ char* kbuf(int i) const { return lds + (i & 1) * L::KBYTES; }
  __device__ __forceinline__ char* vbuf(int i) const {
    return lds + 2 * L::KBYTES + (i & 1) * L::VBYTES;
  }
  __device__ __forceinline__ int kb(int i) const { return key_begin + i * KN; }
  __device__ __forceinline__ int nvalid(int i) const { return min(KN, key_end - kb(i)); }
  __device__ __forceinline__ bool masked(int i) const {
    return kb(i) + KN > key_end || kb(i) + KN - 1 > diag_from;
  }
  // global -> registers: the subtile staged at half-step h
  __device__ __forceinline__ void stage_load(TileRegs<D>& r, int h) {
    const bool isv = h & 1;
    const int t = min(isv ? h / 2 : h / 2 + 1, nsub - 1);
    tile_load<D>(r, to, (isv ? vbase : kbase) + (size_t)kb(t) * rs, rs, nvalid(t));
  }
  // registers -> LDS: chunk c of the subtile staged at half-step h
  __device__ __forceinline__ void stage_store(const TileRegs<D>& r, int c, int h) {
    constexpr bool kAllThreads = (KN * TileRegs<D>::CPR) % kAttnThreads == 0;
    const int ci = threadIdx.x + c * kAttnThreads;
    if (kAllThreads || ci < KN * TileRegs<D>::CPR) {
      const int row = ci / TileRegs<D>::CPR, col = (ci % TileRegs<D>::CPR) * 16;
      const bool isv = h & 1;
      char* dst = isv ? vbuf(h / 2) + row * L::VS : kbuf(h / 2 + 1) + row * L::KS;
      *reinterpret_cast<u32x4_t*>(dst + col) = r.c[c];
    }
  }
  // the staging work of a phase, spread over its MFMA slots: the stores of the
  // subtile for half-step h, then the loads for half-step h + 2 into the same registers
  template <int BANK>
  __device__ __forceinline__ void stage_slot(int j, int h) {
    if (j < NC) stage_store(bank[BANK], j, h);
    else if (j == NC) stage_load(bank[BANK], h + 2);
  }

  __device__ __forceinline__ static int k_off(int j) {
    return (j / KSTEPS) * 32 * L::KS + (j % KSTEPS) * 32;
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

  // Phase A(i) (EXP) or P (!EXP, i = -1): QK^T of subtile i+1 into nxt (when NEXT) and
  // exp/sum/pack of cur into pb, next to the staging of half-step h.
  template <bool NEXT, bool EXP, int BANK>
  __device__ __forceinline__ void phase_a(WaveState<D, QT>& st, const Scores& cur,
                                          Scores& nxt, POps& pb, int i, int h) {
    const int lane = threadIdx.x & 63, n = lane & 31, hf = lane >> 5;
    constexpr int EPS = 16 * NH / NQK;  // exp elements per slot and query tile
    static_assert(EPS * NQK == 16 * NH && 8 % EPS == 0, "the exps split evenly over slots");
    const char* kp = kbuf(i + 1) + n * L::KS + hf * 16;
    bf16x8_t ka[NQK];
    if (NEXT) {
#pragma unroll
      for (int j = 0; j < PFK; ++j)
        ka[j] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(kp + k_off(j)));
    }
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
        if (j + PFK < NQK)
          ka[j + PFK] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(kp + k_off(j + PFK)));
        const int kk = j / KSTEPS, ks = j % KSTEPS;
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
          nxt[kk][qt] = mfma32x32x16(ka[j], st.q[qt][ks], ks == 0 ? zero : nxt[kk][qt]);
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
      stage_slot<BANK>(j, h);
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

  // Phase B(i): O^T += V^T P^T for subtile i next to the mask and row max of nxt
  // (subtile i+1, when NEXT), then the rescale decision; staging of half-step h.
  template <bool NEXT, int BANK>
  __device__ __forceinline__ void phase_b(WaveState<D, QT>& st, Scores& nxt, const POps& pb,
                                          int i, int h, const int (&tpos)[QT]) {
    const int lane = threadIdx.x & 63, hf = lane >> 5;
    if (NEXT && masked(i + 1)) mask_scores(nxt, i + 1, tpos);
    const char* vp = vbuf(i) + (4 * hf + ((lane & 15) >> 2)) * L::VS +
                     (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;
    u32x4_t va[NPV];
    auto vread = [&](int j) {
      const int ks = j / (D / 32), dt = j % (D / 32);
      const u32x2_t lo = lds_read_tr16(vp + (16 * ks) * L::VS + dt * 64);
      const u32x2_t hi = lds_read_tr16(vp + (16 * ks + 8) * L::VS + dt * 64);
      return u32x4_t{lo[0], lo[1], hi[0], hi[1]};
    };
#pragma unroll
    for (int j = 0; j < PFV; ++j) va[j] = vread(j);
    constexpr int MPS = 16 * NH / NPV;  // max elements per slot and query tile
    static_assert(MPS * NPV == 16 * NH, "the row max splits evenly over the PV slots");
    float mx[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) mx[qt] = -INFINITY;
#pragma unroll
    for (int j = 0; j < NPV; ++j) {
      if (j + PFV < NPV) va[j + PFV] = vread(j + PFV);
      const int ks = j / (D / 32), dt = j % (D / 32);
#pragma unroll
      for (int qt = 0; qt < QT; ++qt)
        st.o[qt][dt] = mfma32x32x16(as_bf16x8(va[j]), pb[qt][ks], st.o[qt][dt]);
      if (NEXT) {
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
#pragma unroll
          for (int e = 0; e < MPS; ++e) {
            const int x = j * MPS + e;
            mx[qt] = fmaxf(mx[qt], nxt[x >> 4][qt][x & 15]);
          }
      }
      stage_slot<BANK>(j, h);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (NEXT) {
      float mxs[QT];
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) mxs[qt] = pair_max(mx[qt]) * sl;
      rescale(st, mxs);
    }
  }

  // A(i) then B(i), cur = S(i), nxt = S(i+1); phases 2i+1 and 2i+2
  template <bool NEXT>
  __device__ __forceinline__ void step(WaveState<D, QT>& st, const Scores& cur, Scores& nxt,
                                       POps& pb, int i, const int (&tpos)[QT]) {
    phase_a<NEXT, true, 1>(st, cur, nxt, pb, i, 2 * i + 1 + grp);
    __syncthreads();
    phase_b<NEXT, 0>(st, nxt, pb, i, 2 * i + 2 + grp, tpos);
    __syncthreads();
  }

  // The first loads, which depend on nothing the caller computes, issued before the
  // caller's query loads so that their latencies overlap: K(0), and for group 0 the
  // subtile of its half-step 1 (V(0)), for group 1 that of half-step 0 (K(1)), which
  // it stages in the prologue because it waits that half-step out.
  __device__ __forceinline__ void begin() {
    to.init(rs);
    nsub = (key_end - key_begin + KN - 1) / KN;
    tile_load<D>(bank[0], to, kbase + (size_t)kb(0) * rs, rs, nvalid(0));
    stage_load(bank[1], grp ? 0 : 1);
  }

  __device__ __forceinline__ void run(WaveState<D, QT>& st, const int (&tpos)[QT]) {
    // prologue: K(0) into LDS (and K(1) for group 1), then the registers of the first
    // two phases: the subtiles of half-steps grp and grp + 1
    tile_store<D, L::KS>(bank[0], kbuf(0));
    if (grp) {
      for (int c = 0; c < NC; ++c) stage_store(bank[1], c, 0);
      stage_load(bank[0], 1);
      stage_load(bank[1], 2);
    } else {
      stage_load(bank[0], 0);
    }
    __syncthreads();
    if (grp) __syncthreads();            // group 1 trails by one half-step
    Scores sa, sb;
    POps pb;
    phase_a<true, false, 0>(st, sa, sa, pb, -1, grp);   // P
    max_all(st, sa, 0, tpos);
    __syncthreads();
    int i = 0;
    for (; i + 2 < nsub; i += 2) {
      step<true>(st, sa, sb, pb, i, tpos);
      step<true>(st, sb, sa, pb, i + 1, tpos);
    }
    if (i + 1 < nsub) {
      step<true>(st, sa, sb, pb, i, tpos);
      step<false>(st, sb, sa, pb, i + 1, tpos);
    } else {
      step<false>(st, sa, sb, pb, i, tpos);
    }
    if (!grp) __syncthreads();           // group 0's share of the last half-step
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
  w.lds = lds;
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
  w.run(st, tpos);
}

// normalise and store one query tile's partial: o rounded to bf16 (nearest even) [D],
// lse (natural log) in fp32
template <int D, int QT>
__device__ __forceinline__ void store_partial(const WaveState<D, QT>& st, int qt, bool valid,
                                              uint16_t* __restrict__ po, float* __restrict__ pl) {
  const int lane = threadIdx.x & 63, hf = lane >> 5;
  const float ltot = pair_sum(st.l[qt]);
  if (!valid) return;
  const float inv = 1.f / ltot;
  // lane (n, hf) holds dims dt*32 + ii*8 + hf*4 + r of its row; they are stored as
  // the contiguous half hf of the row (position hf*D/2 + dt*16 + ii*4 + r), so each
  // lane writes, and the merge reads, whole 16-byte chunks
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int i2 = 0; i2 < 2; ++i2) {
      const f32x16_t& o = st.o[qt][dt];
      const int a = 8 * i2;
      const u32x4_t w = {pack_bf16x2(o[a] * inv, o[a + 1] * inv),
                         pack_bf16x2(o[a + 2] * inv, o[a + 3] * inv),
                         pack_bf16x2(o[a + 4] * inv, o[a + 5] * inv),
                         pack_bf16x2(o[a + 6] * inv, o[a + 7] * inv)};
      *reinterpret_cast<u32x4_t*>(po + hf * (D / 2) + dt * 16 + i2 * 8) = w;
    }
  if (hf == 0) *pl = (st.m[qt] + __log2f(ltot)) * 0.69314718055994530942f;
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
  // The parts are read CH at a time so that their loads are in flight together;
  // indices past nh are clamped to the row's last part and given weight 0.
#ifndef MOBA_MERGE_CH
#define MOBA_MERGE_CH 4
#endif
  constexpr int CH = MOBA_MERGE_CH;
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
    u32x4_t x[CH][D / 16];     // the lane's half of each part row (see store_partial)
    float w[CH];
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const int sc = min(s0 + u, nh - 1);
      const uint16_t* ps = po + (size_t)sc * D + hf * (D / 2);
#pragma unroll
      for (int c = 0; c < D / 16; ++c) x[u][c] = *reinterpret_cast<const u32x4_t*>(ps + c * 8);
      w[u] = s0 + u < nh ? expf(pl[(size_t)sc * ls] - L) : 0.f;
    }
#pragma unroll
    for (int u = 0; u < CH; ++u)
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const u32x4_t& xc = x[u][dt * 2 + ii / 2];
          const u32x2_t y = {xc[(ii & 1) * 2], xc[(ii & 1) * 2 + 1]};
          const float xf[4] = {__uint_as_float(y[0] << 16), __uint_as_float(y[0] & 0xffff0000u),
                               __uint_as_float(y[1] << 16), __uint_as_float(y[1] & 0xffff0000u)};
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[dt][ii][r] = fmaf(w[u], xf[r], acc[dt][ii][r]);
        }
  }
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

  // entry of this lane's row in group rg, and that row's query operands
  auto entry_of = [&](int rg) -> uint32_t {
    const int e = tl.y + rg * 32 + n;
    return (rg < ngroups && e < tl.z) ? entries[e] : 0xffffffffu;
  };
  auto load_qops = [&](uint32_t ent, bf16x8_t (&bq)[KS]) {
    const bool valid = ent != 0xffffffffu;
    const int rr = valid ? (int)(ent >> sb) : 0;
    const uint16_t* qrow = q + ((size_t)((size_t)tok0 + rr / G) * hq + g * G + rr % G) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4_t x = {0u, 0u, 0u, 0u};
      if (valid) x = *reinterpret_cast<const u32x4_t*>(qrow + 16 * ks + 8 * hf);
      bq[ks] = as_bf16x8(x);
    }
  };

  // One 32-row group with query operands bq: scores, softmax, P V, partial store.
  // `refill` runs right after the QK MFMAs, when bq is free: it loads a later group's
  // query rows into bq.
  auto group = [&](int rg, uint32_t ent_cur, bf16x8_t (&bq)[KS], auto&& refill) {
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
    store_partial(st, 0, valid, part_o + (row * (topk - 1) + slot) * D,
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
                               const int4* tiles, const int32_t* tile_count,
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
