// Full-attention decode after a prefill: n new query tokens, which are the last n
// positions of the key sequence, attend every key up to their own position.  After a
// MoBA prefill, generation switches to full attention ("MoBA: Mixture of Block
// Attention for Long-Context LLMs", paper summary page, "Limitations"; README bullet
// "Seamlessly Transition between Full and Sparse Attention").
//
// HBM-bound: every key and value of the cache is read once per 32 query rows.  The
// G*n query rows of a kv-head (G query heads per kv-head, n new tokens) form 32-row
// MFMA tiles (one for decode: G*n <= 32), so each key row read serves a whole tile.  The key range is split over many
// single-wavefront workgroups (split-K), each writing an fp32 (o, lse) partial for its
// rows; a second kernel merges the partials by log-sum-exp.
//
// Per 32-key subtile a wavefront reads the K rows straight into MFMA A operands
// (lane = key), computes S^T = K Q^T (v_mfma_f32_32x32x16_bf16, lane = query), runs
// the online softmax in the log2 domain, stages the V rows in LDS and reads V^T with
// the transpose read ds_read_b64_tr_b16 in the key order the score registers hold, so
// that O^T += V^T P^T takes P^T straight from registers.  The next subtile's loads are
// in flight while one is computed.
#include "moba_internal.h"

namespace moba {
namespace {

constexpr int kDecMaxRows = 1024;     // query rows per kv-head (32 per MFMA tile)
constexpr int kDecTargetWaves = 2048; // split the keys until about this many wavefronts

typedef short dec_s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) dec_s16x4_t dec_lds_s16x4_t;

// within each group of 16 lanes, lane i receives element i%4 of the 8 bytes addressed
// by lanes 4j + i/4, j = 0..3
__device__ __forceinline__ u32x2_t dec_tr16(const char* p) {
  const dec_s16x4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((dec_lds_s16x4_t*)(p));
  return __builtin_bit_cast(u32x2_t, r);
}

__device__ __forceinline__ float dec_pair_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                  false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float dec_pair_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                  false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// One wavefront: the 32 rows rg*32 .. of the rows r = i*G + hl (new token i, query head
// g*G + hl) of kv-head g of sequence b, blockIdx.y = g * RG + rg, against 32-key subtiles
// [s*spt, min((s+1)*spt, nsub)).
template <int D>
__global__ __launch_bounds__(64, 2) void decode_split_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, int n, int Tk, int hq, int hkv, float sl, int spt,
    float* __restrict__ part_o, float* __restrict__ part_lse) {
  constexpr int KS = D / 16;           // MFMA k-steps over the head dim
  constexpr int VS = 2 * D + 64;       // V row stride in LDS: transpose reads hit all banks
  constexpr int CPR = D / 8;           // 16-byte chunks per row
  constexpr int CPL = 32 * CPR / 64;   // V chunks per lane per subtile
  __shared__ __attribute__((aligned(16))) char vt[32 * VS];
  const int s = blockIdx.x, b = blockIdx.z, nsplit = gridDim.x;
  const int lane = threadIdx.x, n32 = lane & 31, hf = lane >> 5;
  const int G = hq / hkv, R = G * n, RG = (R + 31) / 32;
  const int g = blockIdx.y / RG, r = (blockIdx.y % RG) * 32 + n32;
  const bool rv = r < R;
  const int i = rv ? r / G : 0, hl = rv ? r % G : 0;
  const int pos = Tk - n + i;          // this row's position among the keys

  // Q^T operand: query n32, dims 16ks + 8hf .. +7 (zero for padding rows)
  bf16x8_t bq[KS];
  const uint16_t* qrow = q + (((size_t)b * n + i) * hq + g * G + hl) * D;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    u32x4_t x = {0u, 0u, 0u, 0u};
    if (rv) x = *reinterpret_cast<const u32x4_t*>(qrow + 16 * ks + 8 * hf);
    bq[ks] = as_bf16x8(x);
  }
  const size_t rs = (size_t)hkv * D;   // elements between consecutive keys
  const uint16_t* kbase = k + ((size_t)b * Tk * hkv + g) * D;
  const uint16_t* vbase = v + ((size_t)b * Tk * hkv + g) * D;
  const int nsub = (Tk + 31) / 32;
  const int sub0 = s * spt, sub1 = min(sub0 + spt, nsub);

  float m = -INFINITY, l = 0.f;
  f32x16_t o[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[dt][e] = 0.f;
  // V^T read address of this lane (key order matching the score registers)
  const char* vp = vt + (4 * hf + ((lane & 15) >> 2)) * VS +
                   (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;

  // global -> registers: the K operands (lane = key) or this lane's V chunks of a
  // subtile; rows past the end of the cache read as zeros (and are masked)
  auto rsrc = [&](const uint16_t* base, int kb) {
    const int bytes = (int)(min(32, Tk - kb) * rs * sizeof(uint16_t));
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base + (size_t)kb * rs),
                                             (short)0, bytes, 0x00020000);
  };
  auto load_k = [&](int sub, u32x4_t (&ka)[KS]) {
    const __amdgpu_buffer_rsrc_t rk = rsrc(kbase, sub * 32);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      ka[ks] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                               rk, (int)((n32 * rs + 16 * ks + 8 * hf) * 2), 0, 0));
  };
  auto load_v = [&](int sub, u32x4_t (&vc)[CPL]) {
    const __amdgpu_buffer_rsrc_t rvv = rsrc(vbase, sub * 32);
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int x = lane + 64 * c;
      vc[c] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                              rvv, (int)(((x / CPR) * rs + (x % CPR) * 8) * 2), 0, 0));
    }
  };
  // subtile sub from K operands ka and V chunks vc; once vc is in LDS, the V chunks of
  // subtile vnext (when in range) are loaded into it
  auto compute = [&](int sub, const u32x4_t (&ka)[KS], u32x4_t (&vc)[CPL], int vnext) {
    const int kb = sub * 32;
    // the previous subtile's V^T reads are complete (their MFMAs have issued): rewrite
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int x = lane + 64 * c;
      *reinterpret_cast<u32x4_t*>(vt + (x / CPR) * VS + (x % CPR) * 16) = vc[c];
    }
    if (vnext < sub1) load_v(vnext, vc);
    // S^T = K Q^T: lane holds query n32, keys (e/4)*8 + hf*4 + e%4
    f32x16_t sc = {};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) sc = mfma32x32x16(as_bf16x8(ka[ks]), bq[ks], sc);
    if (kb + 31 > Tk - n) {            // some row does not see every key of the subtile
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (kb + (e >> 2) * 8 + hf * 4 + (e & 3) > pos) sc[e] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sc[e]);
    const float mnew = fmaxf(m, dec_pair_max(mx) * sl);
    const float mref = mnew == -INFINITY ? 0.f : mnew;
    const float alpha = __builtin_amdgcn_exp2f(m - mref);   // 0 while m = -inf
    m = mnew;
    l *= alpha;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[dt][e] *= alpha;
    float p[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      p[e] = __builtin_amdgcn_exp2f(fmaf(sc[e], sl, -mref));
      l += p[e];
    }
    bf16x8_t pb[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(p[8 * h + 2 * e], p[8 * h + 2 * e + 1]);
      pb[h] = as_bf16x8(u32x4_t{w[0], w[1], w[2], w[3]});
    }
    // O^T += V^T P^T over the subtile's two 16-key k-steps
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        const u32x2_t lo = dec_tr16(vp + (16 * ks) * VS + dt * 64);
        const u32x2_t hi = dec_tr16(vp + (16 * ks + 8) * VS + dt * 64);
        o[dt] = mfma32x32x16(as_bf16x8(u32x4_t{lo[0], lo[1], hi[0], hi[1]}), pb[ks], o[dt]);
      }
  };
  // the next subtile's K (second register set) and V (reloaded into the V registers
  // once they are in LDS) are in flight while one subtile is computed
  u32x4_t ka0[KS], ka1[KS], vc[CPL];
  if (sub0 < sub1) {
    load_k(sub0, ka0);
    load_v(sub0, vc);
  }
  for (int sub = sub0; sub < sub1; sub += 2) {
    if (sub + 1 < sub1) load_k(sub + 1, ka1);
    compute(sub, ka0, vc, sub + 1);
    if (sub + 1 >= sub1) break;
    if (sub + 2 < sub1) load_k(sub + 2, ka0);
    compute(sub + 1, ka1, vc, sub + 2);
  }

  // partial of this split: o normalised (fp32), lse in natural log; a row that saw no
  // key of the split gets lse = -inf and o = 0
  const float ltot = dec_pair_sum(l);
  if (!rv) return;
  const size_t pr = ((size_t)(b * hkv + g) * nsplit + s) * R + r;
  const bool seen = ltot > 0.f;
  const float inv = seen ? 1.f / ltot : 0.f;
  float* po = part_o + pr * D + hf * 4;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const f32x4_t w = {o[dt][ii * 4] * inv, o[dt][ii * 4 + 1] * inv,
                         o[dt][ii * 4 + 2] * inv, o[dt][ii * 4 + 3] * inv};
      *reinterpret_cast<f32x4_t*>(po + dt * 32 + ii * 8) = w;
    }
  if (hf == 0)
    part_lse[pr] = seen ? (m + __log2f(ltot)) * 0.69314718055994530942f : -INFINITY;
}

// One workgroup per (row, kv-head, sequence): the log-sum-exp merge of the row's split
// partials, written as bf16 out (nearest even) and fp32 lse.  Thread t reads dims
// 4*(t % (D/4)) .. +3 of splits t / (D/4), t / (D/4) + GROUPS, ..., kMergeBatch at a
// time; the split groups are then summed through LDS in a fixed order.
constexpr int kMergeThreads = 1024;
constexpr int kMergeBatch = 8;         // splits whose loads a thread issues together

template <int D>
__global__ __launch_bounds__(kMergeThreads) void decode_merge_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_lse, int n, int hq,
    int hkv, int nsplit, uint16_t* __restrict__ out, float* __restrict__ lse) {
  constexpr int LANES = D / 4, GROUPS = kMergeThreads / LANES;
  __shared__ float red[kMergeThreads];
  __shared__ f32x4_t racc[kMergeThreads];
  const int r = blockIdx.x, g = blockIdx.y, b = blockIdx.z, t = threadIdx.x;
  const int G = hq / hkv, R = G * n;
  const int i = r / G, h = g * G + r % G;
  const size_t p0 = (size_t)(b * hkv + g) * nsplit * R + r;   // split s: p0 + s * R
  // the largest split lse of the row
  float mx = -INFINITY;
  for (int s = t; s < nsplit; s += kMergeThreads) mx = fmaxf(mx, part_lse[p0 + (size_t)s * R]);
  red[t] = mx;
  __syncthreads();
  for (int w = kMergeThreads / 2; w > 0; w >>= 1) {
    if (t < w) red[t] = fmaxf(red[t], red[t + w]);
    __syncthreads();
  }
  mx = red[0];
  __syncthreads();
  const int c4 = t % LANES, sg = t / LANES;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  for (int s0 = sg; s0 < nsplit; s0 += GROUPS * kMergeBatch) {
    float ls[kMergeBatch];
    f32x4_t x[kMergeBatch];
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      const int s = s0 + u * GROUPS;
      ls[u] = s < nsplit ? part_lse[p0 + (size_t)s * R] : -INFINITY;
    }
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      const int s = s0 + u * GROUPS;
      // a split that saw no key of this row (lse = -inf) has weight 0
      x[u] = ls[u] != -INFINITY ? *reinterpret_cast<const f32x4_t*>(
                                      part_o + (p0 + (size_t)s * R) * D + 4 * c4)
                                : f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      const float w = ls[u] != -INFINITY ? expf(ls[u] - mx) : 0.f;
      den += w;
      acc += w * x[u];
    }
  }
  red[t] = den;
  racc[t] = acc;
  __syncthreads();
  if (sg != 0) return;
  for (int q2 = 1; q2 < GROUPS; ++q2) {
    den += red[q2 * LANES + c4];
    acc += racc[q2 * LANES + c4];
  }
  const float inv = 1.f / den;
  uint16_t* orow = out + (((size_t)b * n + i) * hq + h) * D + 4 * c4;
  const u32x2_t pk = {f32_to_bf16_rne(acc[0] * inv) | (f32_to_bf16_rne(acc[1] * inv) << 16),
                      f32_to_bf16_rne(acc[2] * inv) | (f32_to_bf16_rne(acc[3] * inv) << 16)};
  *reinterpret_cast<u32x2_t*>(orow) = pk;
  if (c4 == 0) lse[((size_t)b * hq + h) * n + i] = mx + logf(den);
}

}  // namespace

DecodePlan decode_plan(int b, int n, int Tk, int hq, int hkv, int d) {
  DecodePlan p{};
  const int nsub = (Tk + 31) / 32;
  const long groups = (long)b * hkv * ((hq / hkv * n + 31) / 32);   // row tiles
  int nsplit = (int)((kDecTargetWaves + groups - 1) / groups);
  if (nsplit > nsub) nsplit = nsub;
  if (nsplit < 1) nsplit = 1;
  p.spt = (nsub + nsplit - 1) / nsplit;
  p.nsplit = (nsub + p.spt - 1) / p.spt;
  const size_t rows = (size_t)b * hkv * p.nsplit * (hq / hkv) * n;
  p.part_o_bytes = rows * d * sizeof(float);
  p.part_lse_bytes = rows * sizeof(float);
  return p;
}

int decode_max_rows() { return kDecMaxRows; }

hipError_t launch_decode(int b, int n, int Tk, int hq, int hkv, int d, float scale,
                         const DecodePlan& p, const uint16_t* q, const uint16_t* k,
                         const uint16_t* v, float* part_o, float* part_lse, uint16_t* out,
                         float* lse, hipStream_t st) {
  const float sl = scale * 1.4426950408889634f;
  const int RG = ((hq / hkv) * n + 31) / 32;
  const dim3 grid((unsigned)p.nsplit, (unsigned)(hkv * RG), (unsigned)b);
  const dim3 mgrid((unsigned)((hq / hkv) * n), (unsigned)hkv, (unsigned)b);
  if (d == 128) {
    hipLaunchKernelGGL((decode_split_kernel<128>), grid, dim3(64), 0, st, q, k, v, n, Tk, hq,
                       hkv, sl, p.spt, part_o, part_lse);
    hipLaunchKernelGGL((decode_merge_kernel<128>), mgrid, dim3(kMergeThreads), 0, st, part_o,
                       part_lse, n, hq, hkv, p.nsplit, out, lse);
  } else {
    hipLaunchKernelGGL((decode_split_kernel<64>), grid, dim3(64), 0, st, q, k, v, n, Tk, hq,
                       hkv, sl, p.spt, part_o, part_lse);
    hipLaunchKernelGGL((decode_merge_kernel<64>), mgrid, dim3(kMergeThreads), 0, st, part_o,
                       part_lse, n, hq, hkv, p.nsplit, out, lse);
  }
  return hipGetLastError();
}

}  // namespace moba
