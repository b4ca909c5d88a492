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
//            (converted to bf16), A = V^T from LDS.  V is transposed while it is
//            staged, with the keys of each 16-key group stored in the order the
//            score registers hold them, so no register shuffle is needed.
// Online softmax in the log2 domain (scale * log2(e) folded into one FMA).
#include "moba_internal.h"

namespace moba {

constexpr int KN = 64;  // keys per LDS subtile

template <int D>
__device__ __forceinline__ int k_lds_off(int key, int chunk) {
  return key * (D * 2) + ((chunk ^ (key & 7)) << 4);
}
__device__ __forceinline__ int v_lds_off(int dim, int chunk) {
  return dim * (KN * 2) + ((chunk ^ ((dim ^ (dim >> 3)) & 7)) << 4);
}

template <int D, int QT>
struct WaveState {
  bf16x8_t q[QT][D / 16];
  f32x16_t o[QT][D / 32];
  float m[QT], l[QT];
};

// keys [key0, key0 + nvalid) of kv-head row stride `rs` -> LDS (zeros past nvalid)
template <int D>
__device__ __forceinline__ void stage_kv(char* lk, char* lv, const uint16_t* __restrict__ kp,
                                         const uint16_t* __restrict__ vp, size_t rs,
                                         int nvalid) {
  constexpr int CPR = D / 8;
  const int tid = threadIdx.x;
  const u32x4_t zero = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int ci = tid; ci < KN * CPR; ci += kThreads) {
    const int key = ci / CPR, ch = ci % CPR;
    u32x4_t x = zero;
    if (key < nvalid) x = *reinterpret_cast<const u32x4_t*>(kp + key * rs + ch * 8);
    *reinterpret_cast<u32x4_t*>(lk + k_lds_off<D>(key, ch)) = x;
  }
#pragma unroll
  for (int combo = tid; combo < (KN / 4) * CPR; combo += kThreads) {
    const int kq = combo / CPR, dc = combo % CPR;
    u32x4_t rows[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int key = 4 * kq + e;
      rows[e] = zero;
      if (key < nvalid) rows[e] = *reinterpret_cast<const u32x4_t*>(vp + key * rs + dc * 8);
    }
    // keys 4kq..4kq+3 sit at permuted positions pos..pos+3 of their 16-key group:
    // groups of four keys are stored in the order 0, 2, 1, 3
    const int grp = kq & 3;
    const int pos = (kq >> 2) * 16 + (((grp & 1) << 1) | (grp >> 1)) * 4;
    const int chunk = pos >> 3, sub = (pos & 7) * 2;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t lo01 = __builtin_amdgcn_perm(rows[1][i], rows[0][i], 0x05040100u);
      const uint32_t lo23 = __builtin_amdgcn_perm(rows[3][i], rows[2][i], 0x05040100u);
      const uint32_t hi01 = __builtin_amdgcn_perm(rows[1][i], rows[0][i], 0x07060302u);
      const uint32_t hi23 = __builtin_amdgcn_perm(rows[3][i], rows[2][i], 0x07060302u);
      const int dim = dc * 8 + 2 * i;
      *reinterpret_cast<u32x2_t*>(lv + v_lds_off(dim, chunk) + sub) = u32x2_t{lo01, lo23};
      *reinterpret_cast<u32x2_t*>(lv + v_lds_off(dim + 1, chunk) + sub) = u32x2_t{hi01, hi23};
    }
  }
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

// one 64-key subtile staged in LDS.  nkeys: valid keys; causal: mask key > tpos.
template <int D, int QT>
__device__ __forceinline__ void attend_subtile(WaveState<D, QT>& st, const char* lk,
                                               const char* lv, float sl, int nkeys,
                                               bool causal, int kb, const int (&tpos)[QT]) {
  const int lane = threadIdx.x & 63, n = lane & 31, hf = lane >> 5;
  f32x16_t s[2][QT];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kk][qt][i] = 0.f;
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const bf16x8_t a = as_bf16x8(
          *reinterpret_cast<const u32x4_t*>(lk + k_lds_off<D>(kk * 32 + n, 2 * ks + hf)));
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) s[kk][qt] = mfma32x32x16(a, st.q[qt][ks], s[kk][qt]);
    }
  }
  const bool need_mask = causal || nkeys < KN;
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    if (need_mask) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kr = kk * 32 + (i >> 2) * 8 + hf * 4 + (i & 3);
          const bool ok = kr < nkeys && (!causal || kb + kr <= tpos[qt]);
          if (!ok) s[kk][qt][i] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kk][qt][i]);
    mx = fmaxf(mx, xor32_f32(mx));
    const float mnew = fmaxf(st.m[qt], mx * sl);
    const float mref = (mnew == -INFINITY) ? 0.f : mnew;
    const float alpha = __builtin_amdgcn_exp2f(st.m[qt] - mref);
    float rs = 0.f;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[kk][qt][i], sl, -mref));
        s[kk][qt][i] = p;
        rs += p;
      }
    st.l[qt] = st.l[qt] * alpha + rs;
    st.m[qt] = mnew;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) st.o[qt][dt][i] *= alpha;
  }
  bf16x8_t pb[QT][4];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const f32x16_t& v = s[ks >> 1][qt];
      const int o = 8 * (ks & 1);
      u32x4_t w;
      w[0] = pack_bf16x2(v[o + 0], v[o + 1]);
      w[1] = pack_bf16x2(v[o + 2], v[o + 3]);
      w[2] = pack_bf16x2(v[o + 4], v[o + 5]);
      w[3] = pack_bf16x2(v[o + 6], v[o + 7]);
      pb[qt][ks] = as_bf16x8(w);
    }
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8_t a = as_bf16x8(
          *reinterpret_cast<const u32x4_t*>(lv + v_lds_off(dt * 32 + n, 2 * ks + hf)));
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) st.o[qt][dt] = mfma32x32x16(a, pb[qt][ks], st.o[qt][dt]);
    }
  }
}

// normalise and store one query tile's partial (o fp32 [D], lse natural log)
template <int D, int QT>
__device__ __forceinline__ void store_partial(const WaveState<D, QT>& st, int qt, bool valid,
                                              float* __restrict__ po, float* __restrict__ pl) {
  const int lane = threadIdx.x & 63, hf = lane >> 5;
  const float ltot = st.l[qt] + xor32_f32(st.l[qt]);
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
template <int D, int QT>
__global__ __launch_bounds__(kThreads) void attn_history_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, int T, int hq, int hkv, int block, int topk,
    float sl, int g0, int ng, int nb, const int4* __restrict__ tiles,
    const int32_t* __restrict__ tile_count, const uint32_t* __restrict__ entries,
    float* __restrict__ part_o, float* __restrict__ part_lse) {
  __shared__ __attribute__((aligned(16))) char lk[KN * D * 2];
  __shared__ __attribute__((aligned(16))) char lv[D * KN * 2];
  const int tile_id = blockIdx.x;
  if (tile_id >= *tile_count) return;
  const int4 tl = tiles[tile_id];
  const int list = tl.x;
  const int j = list % nb, gi = (list / nb) % ng, b = list / (nb * ng);
  const int G = hq / hkv, g = g0 + gi;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, n = lane & 31;

  WaveState<D, QT> st;
  int tq[QT], hlq[QT], slq[QT];
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
    const uint16_t* qrow = q + ((size_t)((size_t)b * T + tq[qt]) * hq + g * G + hlq[qt]) * D;
    load_q(st, qt, qrow, vq[qt]);
  }
  state_init(st);
  const size_t rs = (size_t)hkv * D;
  const int key_begin = j * block, key_end = key_begin + block;
  const uint16_t* kbase = k + ((size_t)b * T * hkv + g) * D;
  const uint16_t* vbase = v + ((size_t)b * T * hkv + g) * D;
  const int dummy[QT] = {};
  for (int kb = key_begin; kb < key_end; kb += KN) {
    const int nvalid = min(KN, key_end - kb);
    __syncthreads();
    stage_kv<D>(lk, lv, kbase + (size_t)kb * rs, vbase + (size_t)kb * rs, rs, nvalid);
    __syncthreads();
    attend_subtile<D, QT>(st, lk, lv, sl, nvalid, false, kb, dummy);
  }
  const int ngq = ng * G;
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const size_t prow = ((size_t)(b * ngq + gi * G + hlq[qt]) * T + tq[qt]) * topk + slq[qt];
    store_partial(st, qt, vq[qt], part_o + prow * D, part_lse + prow);
  }
}

// ---------------------------------------------------------------- current (a5)
// workgroup: 32*QT consecutive tokens of block c, waves = query heads of kv-head g
template <int D, int QT>
__global__ __launch_bounds__(kThreads) void attn_current_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, int T, int hq, int hkv, int block, int topk,
    float sl, int g0, int ng, float* __restrict__ part_o, float* __restrict__ part_lse) {
  __shared__ __attribute__((aligned(16))) char lk[KN * D * 2];
  __shared__ __attribute__((aligned(16))) char lv[D * KN * 2];
  constexpr int TT = 32 * QT;
  const int c = blockIdx.y;
  const int gi = blockIdx.z % ng, b = blockIdx.z / ng;
  const int G = hq / hkv, g = g0 + gi;
  const int t0 = c * block + blockIdx.x * TT;
  const int t_end = min(t0 + TT, (c + 1) * block);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, n = lane & 31;
  const size_t rs = (size_t)hkv * D;
  const uint16_t* kbase = k + ((size_t)b * T * hkv + g) * D;
  const uint16_t* vbase = v + ((size_t)b * T * hkv + g) * D;
  const int ngq = ng * G;
  const int key_begin = c * block;
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
      const uint16_t* qrow =
          q + ((size_t)((size_t)b * T + (vq[qt] ? tpos[qt] : 0)) * hq + g * G + (active ? hl : 0)) * D;
      load_q(st, qt, qrow, vq[qt]);
    }
    state_init(st);
    for (int kb = key_begin; kb < t_end; kb += KN) {
      const int nvalid = min(KN, t_end - kb);
      __syncthreads();
      stage_kv<D>(lk, lv, kbase + (size_t)kb * rs, vbase + (size_t)kb * rs, rs, nvalid);
      __syncthreads();
      if (active) {
        const bool diag = kb + KN - 1 > t0;
        attend_subtile<D, QT>(st, lk, lv, sl, nvalid, diag, kb, tpos);
      }
    }
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
constexpr int kQT = 1;
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
