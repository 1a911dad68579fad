// gfx950 kernels of the graph-transformer block around the edge-aware
// attention layer ("Efficient Edge-aware Attention Network for Graph
// Generation", full-text summary: the new attention replaces the one inside
// a graph transformer, whose block around it is kept). The block as read
// here (the usual block of the denoising graph transformers the method
// builds on):
//   X1 = LN(X + O W_o^T + b_o),  X2 = LN(X1 + W_x2 relu(W_x1 X1 + b_x1) + b_x2)
//   E1 = LN(E'),                 E2 = LN(E1 + W_e2 relu(W_e1 E1 + b_e1) + b_e2)
//   y1 = LN(y + W_yy y + W_yx xbar + W_ye ebar + b_yo), y2 = LN(y1 + W_y2 relu(W_y1 y1 + b_y1) + b_y2)
// with xbar, ebar the means of X2 over real nodes and of E2 over real pairs,
// LN over the feature axis (population variance, eps 1e-5, gain and shift),
// and padded rows / masked pairs of X2 / E2 set to +0.0.
//
// Row layout of the node and edge kernels: a wave takes 16 rows (nodes or
// edge tokens); lane (li, lg) holds, for row li, the features
// f = 16 t + 4 lg + r in v[4 t + r]. A product out^T = W in^T (W [NO, K],
// nn.Linear layout) runs as MFMA tiles with W as the left operand (rows
// o = 16 to + li) and in^T as the right one, both taking the contraction
// indices 16 t + 4 lg + r of their lane: the input rows feed the MFMA from
// registers, and the result D[4 lg + r][li] of tile `to` is feature
// 16 to + 4 lg + r of row li, the same layout again. Layer norms reduce
// in-lane and then over the four lane groups.
#include "ea_device.h"

#include <math.h>

namespace ea {
namespace {

constexpr float kLnEps = 1e-5f;

// Four consecutive elements (one row-layout group) as floats.
template <typename T>
__device__ __forceinline__ void ld4f(float* v, const T* p) {
  if constexpr (sizeof(T) == 2) {
    const u32x2 w = *reinterpret_cast<const u32x2*>(p);
    v[0] = __uint_as_float(w.x << 16); v[1] = __uint_as_float(w.x & 0xffff0000u);
    v[2] = __uint_as_float(w.y << 16); v[3] = __uint_as_float(w.y & 0xffff0000u);
  } else {
    const f32x4 w = *reinterpret_cast<const f32x4*>(p);
    v[0] = w.x; v[1] = w.y; v[2] = w.z; v[3] = w.w;
  }
}
template <typename T>
__device__ __forceinline__ void st4f(T* p, const float* v) {
  if constexpr (sizeof(T) == 2) {
    *reinterpret_cast<u32x2*>(p) = u32x2{pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3])};
  } else {
    *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
  }
}
// Four consecutive elements into dwords w[0 ..] of a fragment.
template <typename T>
__device__ __forceinline__ void ld4w(uint32_t* w, const T* p) {
  if constexpr (sizeof(T) == 2) {
    const u32x2 v = *reinterpret_cast<const u32x2*>(p);
    w[0] = v.x; w[1] = v.y;
  } else {
    const u32x4 v = *reinterpret_cast<const u32x4*>(p);
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  }
}

// Contraction steps over K row-layout features: two groups of four per lane
// and step (Q = 8), or one group when K = 16.
template <int K>
struct Steps {
  static constexpr int NT = K / 16, Q = NT >= 2 ? 8 : 4, NS = NT >= 2 ? NT / 2 : 1;
  static_assert(K % 16 == 0 && (NT == 1 || NT % 2 == 0), "contraction width");
};

// Right-operand fragments of a row-layout vector of K features.
template <typename T, int K>
struct RowIn {
  using S = Steps<K>;
  Frag<T, S::Q> f[S::NS];
  __device__ __forceinline__ void set(const float* v) {  // v[K / 4], rounded to T
#pragma unroll
    for (int s = 0; s < S::NS; ++s) f[s].set(v + s * S::Q);
  }
  __device__ __forceinline__ void load(const T* row, int lg) {  // straight from a row in memory
    constexpr int DW = 4 * (int)sizeof(T) / 4;  // dwords per group of four
#pragma unroll
    for (int s = 0; s < S::NS; ++s) {
      ld4w<T>(f[s].w, row + 32 * s + 4 * lg);
      if constexpr (S::Q == 8) ld4w<T>(f[s].w + DW, row + 32 * s + 16 + 4 * lg);
    }
  }
};

// Left-operand fragment: row o of W [NO, K], step s, in the row-layout order.
template <typename T, int K>
__device__ __forceinline__ Frag<T, Steps<K>::Q> w_frag(const T* W, int o, int s, int lg) {
  using S = Steps<K>;
  constexpr int DW = 4 * (int)sizeof(T) / 4;
  Frag<T, S::Q> a;
  const T* row = W + (size_t)o * K;
  ld4w<T>(a.w, row + 32 * s + 4 * lg);
  if constexpr (S::Q == 8) ld4w<T>(a.w + DW, row + 32 * s + 16 + 4 * lg);
  return a;
}

// out[NO / 4] (row layout) = W in (+ bias), W streamed from memory.
template <typename T, int K, int NO>
__device__ __forceinline__ void row_gemm(float* out, const RowIn<T, K>& in, const T* W, const T* bias, int li,
                                         int lg) {
#pragma unroll
  for (int to = 0; to < NO / 16; ++to) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < Steps<K>::NS; ++s) acc = mma(acc, w_frag<T, K>(W, 16 * to + li, s, lg), in.f[s]);
    float bv[4];
    ld4f<T>(bv, bias + 16 * to + 4 * lg);
#pragma unroll
    for (int r = 0; r < 4; ++r) out[4 * to + r] = acc[r] + bv[r];
  }
}

// In-place layer norm of a row-layout vector of F features (gain g, shift b).
template <typename T, int F>
__device__ __forceinline__ void row_ln(float* v, const T* g, const T* b, int lg) {
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < F / 4; ++k) s += v[k];
  const float mean = lg_sum(s) * (1.f / F);
  float q = 0.f;
#pragma unroll
  for (int k = 0; k < F / 4; ++k) {
    v[k] -= mean;
    q += v[k] * v[k];
  }
  const float inv = 1.f / sqrtf(lg_sum(q) * (1.f / F) + kLnEps);
#pragma unroll
  for (int t = 0; t < F / 16; ++t) {
    float gv[4], bv[4];
    ld4f<T>(gv, g + 16 * t + 4 * lg);
    ld4f<T>(bv, b + 16 * t + 4 * lg);
#pragma unroll
    for (int r = 0; r < 4; ++r) v[4 * t + r] = v[4 * t + r] * inv * gv[r] + bv[r];
  }
}

// ------------------------------------------------------------------ nodes

// Grid (ceil(n / 64), B); wave w takes nodes 64 blockIdx.x + 16 w .. + 15 of
// graph blockIdx.y. Writes X2 and the block's sum of X2 over its real nodes
// (partial_x [B][gridDim.x][D]).
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void blk_node_kernel(BlockArgs k) {
  __shared__ float sum_s[D];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, li = l & 15, lg = l >> 4;
  const int b = blockIdx.y, n = k.n, i = blockIdx.x * 64 + 16 * w + li;
  const bool inr = i < n;
  const size_t row = (size_t)b * n + (inr ? i : 0);
  const bool real = inr && k.mask[row] != 0;
  for (int f = tid; f < D; f += kThreads) sum_s[f] = 0.f;
  auto par = [&](int q) { return static_cast<const T*>(k.p[q]); };
  RowIn<T, D> o_in;
  o_in.load(static_cast<const T*>(k.O) + row * D, lg);
  float x1[D / 4], z[D / 4];
#pragma unroll
  for (int t = 0; t < D / 16; ++t) ld4f<T>(x1 + 4 * t, static_cast<const T*>(k.X) + row * D + 16 * t + 4 * lg);
  row_gemm<T, D, D>(z, o_in, par(kBW_o), par(kBb_o), li, lg);
#pragma unroll
  for (int q = 0; q < D / 4; ++q) x1[q] += z[q];
  row_ln<T, D>(x1, par(kBln_x1_g), par(kBln_x1_b), lg);
  {
    RowIn<T, D> in;
    in.set(x1);
    row_gemm<T, D, D>(z, in, par(kBW_x1), par(kBb_x1), li, lg);
  }
#pragma unroll
  for (int q = 0; q < D / 4; ++q) z[q] = fmaxf(z[q], 0.f);
  {
    RowIn<T, D> in;
    in.set(z);
    row_gemm<T, D, D>(z, in, par(kBW_x2), par(kBb_x2), li, lg);
  }
#pragma unroll
  for (int q = 0; q < D / 4; ++q) z[q] += x1[q];
  row_ln<T, D>(z, par(kBln_x2_g), par(kBln_x2_b), lg);
#pragma unroll
  for (int q = 0; q < D / 4; ++q) z[q] = real ? z[q] : 0.f;
  if (inr) {
#pragma unroll
    for (int t = 0; t < D / 16; ++t) st4f<T>(static_cast<T*>(k.X_out) + row * D + 16 * t + 4 * lg, z + 4 * t);
  }
  __syncthreads();
#pragma unroll
  for (int t = 0; t < D / 16; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) atomicAdd(&sum_s[16 * t + 4 * lg + r], z[4 * t + r]);
  __syncthreads();
  float* part = k.part_x + ((size_t)b * gridDim.x + blockIdx.x) * D;
  for (int f = tid; f < D; f += kThreads) part[f] = sum_s[f];
}

// ------------------------------------------------------------------ edges

// Grid (EX, B): the edge tokens (i, j) of graph blockIdx.y in tiles of 16,
// tile q for wave slot blockIdx.x * 4 + w, stepping by 4 EX. E2 is written
// over E' in place (each lane reads its token's row before writing it).
// Also the block's sum of E2 over its real pairs (partial_e [B][EX][DE]).
template <typename T, int DE>
__global__ __launch_bounds__(kThreads) void blk_edge_kernel(BlockArgs k) {
  constexpr int FE = 2 * DE;
  __shared__ float sum_s[DE];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, li = l & 15, lg = l >> 4;
  const int b = blockIdx.y, n = k.n;
  for (int f = tid; f < DE; f += kThreads) sum_s[f] = 0.f;
  auto par = [&](int q) { return static_cast<const T*>(k.p[q]); };
  // both weights stay in registers for all tiles of the wave
  Frag<T, Steps<DE>::Q> w1[FE / 16][Steps<DE>::NS];
  Frag<T, Steps<FE>::Q> w2[DE / 16][Steps<FE>::NS];
#pragma unroll
  for (int to = 0; to < FE / 16; ++to)
#pragma unroll
    for (int s = 0; s < Steps<DE>::NS; ++s) w1[to][s] = w_frag<T, DE>(par(kBW_e1), 16 * to + li, s, lg);
#pragma unroll
  for (int to = 0; to < DE / 16; ++to)
#pragma unroll
    for (int s = 0; s < Steps<FE>::NS; ++s) w2[to][s] = w_frag<T, FE>(par(kBW_e2), 16 * to + li, s, lg);
  float esum[DE / 4];
#pragma unroll
  for (int q = 0; q < DE / 4; ++q) esum[q] = 0.f;
  T* Eio = static_cast<T*>(k.E_io);
  const int ntok = n * n, ntile = (ntok + 15) / 16;
  for (int tile = blockIdx.x * kWaves + w; tile < ntile; tile += gridDim.x * kWaves) {
    const int tk = 16 * tile + li;
    const bool valid = tk < ntok;
    const int tc = valid ? tk : 0, i = tc / n, j = tc % n;
    const bool real = valid && k.mask[(size_t)b * n + i] != 0 && k.mask[(size_t)b * n + j] != 0;
    T* rowp = Eio + (((size_t)b * n + i) * n + j) * DE;
    float e1[DE / 4], z[DE / 4], h[FE / 4];
#pragma unroll
    for (int t = 0; t < DE / 16; ++t) ld4f<T>(e1 + 4 * t, rowp + 16 * t + 4 * lg);
    row_ln<T, DE>(e1, par(kBln_e1_g), par(kBln_e1_b), lg);
    {
      RowIn<T, DE> in;
      in.set(e1);
#pragma unroll
      for (int to = 0; to < FE / 16; ++to) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < Steps<DE>::NS; ++s) acc = mma(acc, w1[to][s], in.f[s]);
        float bv[4];
        ld4f<T>(bv, par(kBb_e1) + 16 * to + 4 * lg);
#pragma unroll
        for (int r = 0; r < 4; ++r) h[4 * to + r] = fmaxf(acc[r] + bv[r], 0.f);
      }
    }
    {
      RowIn<T, FE> in;
      in.set(h);
#pragma unroll
      for (int to = 0; to < DE / 16; ++to) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < Steps<FE>::NS; ++s) acc = mma(acc, w2[to][s], in.f[s]);
        float bv[4];
        ld4f<T>(bv, par(kBb_e2) + 16 * to + 4 * lg);
#pragma unroll
        for (int r = 0; r < 4; ++r) z[4 * to + r] = acc[r] + bv[r] + e1[4 * to + r];
      }
    }
    row_ln<T, DE>(z, par(kBln_e2_g), par(kBln_e2_b), lg);
#pragma unroll
    for (int q = 0; q < DE / 4; ++q) {
      z[q] = real ? z[q] : 0.f;
      esum[q] += z[q];
    }
    if (valid) {
#pragma unroll
      for (int t = 0; t < DE / 16; ++t) st4f<T>(rowp + 16 * t + 4 * lg, z + 4 * t);
    }
  }
  __syncthreads();
#pragma unroll
  for (int t = 0; t < DE / 16; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) atomicAdd(&sum_s[16 * t + 4 * lg + r], esum[4 * t + r]);
  __syncthreads();
  float* part = k.part_e + ((size_t)b * gridDim.x + blockIdx.x) * DE;
  for (int f = tid; f < DE; f += kThreads) part[f] = sum_s[f];
}

// ------------------------------------------------------------------ y

// One block per graph: the means from the partial sums, then the y path in
// float32 (thread per output feature, loops over the inputs).
template <typename T, int D, int DE>
__global__ __launch_bounds__(kThreads) void blk_y_kernel(BlockArgs k) {
  __shared__ float xbar[D], ebar[DE];
  __shared__ float yv[kMaxBlockDy], y1[kMaxBlockDy], hy[kMaxBlockDy], red[2];
  __shared__ int cnt;
  const int tid = threadIdx.x, b = blockIdx.x, n = k.n, dy = k.dy;
  auto par = [&](int q) { return static_cast<const T*>(k.p[q]); };
  auto P = [&](int q, size_t idx) { return Num<T>::ld(par(q) + idx); };
  if (tid == 0) cnt = 0;
  __syncthreads();
  int c0 = 0;
  for (int i = tid; i < n; i += kThreads) c0 += k.mask[(size_t)b * n + i] != 0;
  atomicAdd(&cnt, c0);
  for (int c = tid; c < dy; c += kThreads) yv[c] = Num<T>::ld(static_cast<const T*>(k.y) + (size_t)b * dy + c);
  __syncthreads();
  const float nr = (float)cnt;
  for (int f = tid; f < D; f += kThreads) {
    float s = 0.f;
    for (int q = 0; q < k.nxb; ++q) s += k.part_x[((size_t)b * k.nxb + q) * D + f];
    xbar[f] = s / fmaxf(nr, 1.f);
  }
  for (int f = tid; f < DE; f += kThreads) {
    float s = 0.f;
    for (int q = 0; q < k.exb; ++q) s += k.part_e[((size_t)b * k.exb + q) * DE + f];
    ebar[f] = s / fmaxf(nr * nr, 1.f);
  }
  __syncthreads();
  // layer norm of v[0 .. dy) in place (gain / shift parameters gq, bq)
  auto block_ln = [&](float* v, int gq, int bq) {
    if (tid == 0) {
      float s = 0.f;
      for (int c = 0; c < dy; ++c) s += v[c];
      const float mean = s / dy;
      float q = 0.f;
      for (int c = 0; c < dy; ++c) q += (v[c] - mean) * (v[c] - mean);
      red[0] = mean;
      red[1] = 1.f / sqrtf(q / dy + kLnEps);
    }
    __syncthreads();
    for (int c = tid; c < dy; c += kThreads) v[c] = (v[c] - red[0]) * red[1] * P(gq, c) + P(bq, c);
    __syncthreads();
  };
  for (int o = tid; o < dy; o += kThreads) {
    float s = yv[o] + P(kBb_yo, o);
    for (int c = 0; c < dy; ++c) s += P(kBW_yy, (size_t)o * dy + c) * yv[c];
    for (int f = 0; f < D; ++f) s += P(kBW_yx, (size_t)o * D + f) * xbar[f];
    for (int f = 0; f < DE; ++f) s += P(kBW_ye, (size_t)o * DE + f) * ebar[f];
    y1[o] = s;
  }
  __syncthreads();
  block_ln(y1, kBln_y1_g, kBln_y1_b);
  for (int o = tid; o < dy; o += kThreads) {
    float s = P(kBb_y1, o);
    for (int c = 0; c < dy; ++c) s += P(kBW_y1, (size_t)o * dy + c) * y1[c];
    hy[o] = fmaxf(s, 0.f);
  }
  __syncthreads();
  for (int o = tid; o < dy; o += kThreads) {
    float s = y1[o] + P(kBb_y2, o);
    for (int c = 0; c < dy; ++c) s += P(kBW_y2, (size_t)o * dy + c) * hy[c];
    yv[o] = s;  // y is no longer needed: y2 takes its place
  }
  __syncthreads();
  block_ln(yv, kBln_y2_g, kBln_y2_b);
  for (int o = tid; o < dy; o += kThreads) Num<T>::st(static_cast<T*>(k.y_out) + (size_t)b * dy + o, yv[o]);
}

template <typename T, int D, int DE>
hipError_t block_shape(const BlockArgs& k, hipStream_t s) {
  hipLaunchKernelGGL((blk_node_kernel<T, D>), dim3(k.nxb, k.B), dim3(kThreads), 0, s, k);
  hipLaunchKernelGGL((blk_edge_kernel<T, DE>), dim3(k.exb, k.B), dim3(kThreads), 0, s, k);
  hipLaunchKernelGGL((blk_y_kernel<T, D, DE>), dim3(k.B), dim3(kThreads), 0, s, k);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_block(const BlockArgs& k, int dtype, int d, int de, hipStream_t s) {
  if (dtype == 1 && d == 256 && de == 64) return block_shape<bf16_t, 256, 64>(k, s);
  if (dtype == 1 && d == 64 && de == 16) return block_shape<bf16_t, 64, 16>(k, s);
  if (dtype == 0 && d == 64 && de == 16) return block_shape<float, 64, 16>(k, s);
  return hipErrorInvalidValue;
}

}  // namespace ea
