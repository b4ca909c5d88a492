// Short convolution of the keys within blocks, before pooling (the FlashMoBA story on
// hyper.ai, paragraph on short convolutions: convolving within blocks clusters the
// relevant information of a block).  Depthwise and causal along tokens, per kv-head
// channel, taps never crossing a block boundary:
//   out[t, g, c] = sum_{i < width, t - i >= start of t's block} w[g, c, i] * k[t - i, g, c]
//
// HBM-bound: every key row is read once and written once.  A thread owns 8 channels
// (16 bytes) of a run of consecutive tokens and slides a window of the last width-1
// rows in registers; neighbouring threads own neighbouring 16-byte chunks of the same
// row, so each row is read and written with whole coalesced lines.
#include "moba_internal.h"

namespace moba {

constexpr int kConvMaxWidth = 8;
constexpr int kConvRun = 64;   // tokens per thread
constexpr int kConvStep = 4;   // rows loaded together

template <int W>
__global__ __launch_bounds__(kThreads) void key_conv_kernel(const uint16_t* __restrict__ k,
                                                            const float* __restrict__ weight,
                                                            SeqMap sq, int cols, int d,
                                                            int block, int runs,
                                                            uint16_t* __restrict__ out) {
  const int chunks = cols / 8;                           // 16-byte chunks per row
  const long gid = (long)blockIdx.x * kThreads + threadIdx.x;
  const int b = blockIdx.y;
  if (gid >= (long)chunks * runs) return;
  const int cc = (int)(gid % chunks), run = (int)(gid / chunks);
  const int T = sq.len(b), tok0 = sq.tok0(b);
  const int t0 = run * kConvRun;
  if (t0 >= T) return;
  const int t1 = min(t0 + kConvRun, T);
  // this chunk's 8 channels: kv-head g, channels c0 .. c0+7
  const int g = (cc * 8) / d, c0 = (cc * 8) % d;
  float wt[W][8];
#pragma unroll
  for (int e = 0; e < 8; ++e)
#pragma unroll
    for (int i = 0; i < W; ++i) wt[i][e] = weight[((size_t)g * d + c0 + e) * W + i];
  const uint16_t* src = k + (size_t)tok0 * cols + cc * 8;
  uint16_t* dst = out + (size_t)tok0 * cols + cc * 8;
  // window: win[i] = row t - i (zero before the block start)
  float win[W][8];
  auto load_row = [&](int t, float (&r)[8]) {
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(src + (size_t)t * cols);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      r[2 * e] = bf16lo(v[e]);
      r[2 * e + 1] = bf16hi(v[e]);
    }
  };
#pragma unroll
  for (int i = 1; i < W; ++i) {
    const int t = t0 - i;
#pragma unroll
    for (int e = 0; e < 8; ++e) win[i][e] = 0.f;
    if (t >= 0 && t / block == t0 / block) load_row(t, win[i]);
  }
  // rows go through in steps of kConvStep: the step's loads are issued together
  for (int ts = t0; ts < t1; ts += kConvStep) {
    u32x4_t rows[kConvStep];     // packed bf16, unpacked when used
#pragma unroll
    for (int u = 0; u < kConvStep; ++u)
      rows[u] = ts + u < t1 ? *reinterpret_cast<const u32x4_t*>(src + (size_t)(ts + u) * cols)
                            : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
    for (int u = 0; u < kConvStep; ++u) {
      const int t = ts + u;
      if (t >= t1) break;
      if (t % block == 0) {        // a block starts: no tap reaches back over it
#pragma unroll
        for (int i = 1; i < W; ++i)
#pragma unroll
          for (int e = 0; e < 8; ++e) win[i][e] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        win[0][2 * e] = bf16lo(rows[u][e]);
        win[0][2 * e + 1] = bf16hi(rows[u][e]);
      }
      uint32_t o[4];
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        float a0 = 0.f, a1 = 0.f;
#pragma unroll
        for (int i = 0; i < W; ++i) {
          a0 = fmaf(wt[i][2 * e2], win[i][2 * e2], a0);
          a1 = fmaf(wt[i][2 * e2 + 1], win[i][2 * e2 + 1], a1);
        }
        o[e2] = f32_to_bf16_rne(a0) | (f32_to_bf16_rne(a1) << 16);
      }
      *reinterpret_cast<u32x4_t*>(dst + (size_t)t * cols) = u32x4_t{o[0], o[1], o[2], o[3]};
      // shift the window: row t becomes tap 1 of row t + 1
#pragma unroll
      for (int i = W - 1; i > 0; --i)
#pragma unroll
        for (int e = 0; e < 8; ++e) win[i][e] = win[i - 1][e];
    }
  }
}

int conv_max_width() { return kConvMaxWidth; }

hipError_t launch_key_conv(const Shape& s, const uint16_t* k, const float* weight, int width,
                           uint16_t* out, hipStream_t st) {
  const int cols = s.hkv * s.d;
  const int runs = (s.T + kConvRun - 1) / kConvRun;
  const long threads = (long)(cols / 8) * runs;
  dim3 grid((unsigned)((threads + kThreads - 1) / kThreads), s.b);
#define MOBA_CONV(WW)                                                                    \
  hipLaunchKernelGGL((key_conv_kernel<WW>), grid, dim3(kThreads), 0, st, k, weight,       \
                     s.seqs(), cols, s.d, s.block, runs, out)
  switch (width) {
    case 1: MOBA_CONV(1); break;
    case 2: MOBA_CONV(2); break;
    case 3: MOBA_CONV(3); break;
    case 4: MOBA_CONV(4); break;
    case 5: MOBA_CONV(5); break;
    case 6: MOBA_CONV(6); break;
    case 7: MOBA_CONV(7); break;
    default: MOBA_CONV(8); break;
  }
#undef MOBA_CONV
  return hipGetLastError();
}

}  // namespace moba
