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

#include <type_traits>

namespace ea {
namespace {

constexpr float kLnEps = 1e-5f;
// Waves per block of the edge kernel: large blocks stage the weights once
// for many token tiles.
constexpr int kEdgeWaves = 4;

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
};

// Fragment in the row-layout contraction order from a row of K elements
// (global memory or LDS): elements 32 s + 4 lg .. + 3 and 32 s + 16 + 4 lg .. + 3.
template <typename T, int K>
__device__ __forceinline__ Frag<T, Steps<K>::Q> frag_at(const T* row, int s, int lg) {
  using S = Steps<K>;
  constexpr int DW = 4 * (int)sizeof(T) / 4;
  Frag<T, S::Q> a;
  ld4w<T>(a.w, row + 32 * s + 4 * lg);
  if constexpr (S::Q == 8) ld4w<T>(a.w + DW, row + 32 * s + 16 + 4 * lg);
  return a;
}

// 16-byte pieces of a [ROWS, COLS] matrix: thread tid takes pieces tid,
// tid + 256, ...; piece q is row q / (COLS / EPC), columns EPC (q % (COLS / EPC)) ..
template <typename T, int ROWS, int COLS, int NT = kThreads>
struct Pieces {
  static constexpr int EPC = 16 / (int)sizeof(T), N = ROWS * COLS / EPC, PER = (N + NT - 1) / NT;
  u32x4 v[PER];
  __device__ __forceinline__ void load(const T* src, int tid) {  // src: row-major, row stride COLS
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int q = tid + e * NT, qc = q < N ? q : 0;
      v[e] = *reinterpret_cast<const u32x4*>(src + (size_t)(qc / (COLS / EPC)) * COLS + EPC * (qc % (COLS / EPC)));
    }
  }
  template <int LD>
  __device__ __forceinline__ void store(T (*dst)[LD], int tid) const {
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int q = tid + e * NT;
      if (PER * NT == N || q < N) *reinterpret_cast<u32x4*>(&dst[q / (COLS / EPC)][EPC * (q % (COLS / EPC))]) = v[e];
    }
  }
};

// A weight matrix [ROWS, COLS] staged in LDS with its columns regrouped so
// that a lane's left-operand fragment is contiguous: column 32 s + 16 h +
// 4 g + r (h < 2, g, r < 4) is stored at 32 s + 8 g + 4 h + r, so the
// contraction values 32 s + 4 lg .. + 3 and 32 s + 16 + 4 lg .. + 3 of lane
// group lg are the 8 elements at 32 s + 8 lg (one 16-byte LDS read). Needs
// COLS a multiple of 32; staged in groups of four elements.
template <typename T, int ROWS, int COLS, int NT>
struct PermStage {
  static_assert(COLS % 32 == 0, "whole steps");
  static constexpr int DW = 4 * (int)sizeof(T) / 4, N = ROWS * COLS / 4, PER = (N + NT - 1) / NT;
  uint32_t v[PER][DW];
  __device__ __forceinline__ void load(const T* src, int tid) {
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int q = tid + e * NT, qc = q < N ? q : 0;
      ld4w<T>(v[e], src + (size_t)(qc / (COLS / 4)) * COLS + 4 * (qc % (COLS / 4)));
    }
  }
  template <int LD>
  __device__ __forceinline__ void store(T (*dst)[LD], int tid) const {
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int q = tid + e * NT;
      if (PER * NT != N && q >= N) continue;
      const int row = q / (COLS / 4), c = 4 * (q % (COLS / 4));
      const int sblk = c / 32, h = (c / 16) & 1, g = (c / 4) & 3;
      T* d = &dst[row][32 * sblk + 8 * g + 4 * h];
      if constexpr (sizeof(T) == 2) *reinterpret_cast<u32x2*>(d) = u32x2{v[e][0], v[e][1]};
      else *reinterpret_cast<u32x4*>(d) = u32x4{v[e][0], v[e][1], v[e][2], v[e][3]};
    }
  }
};

// Left-operand fragment of step s from a row staged by PermStage.
template <typename T, int K>
__device__ __forceinline__ Frag<T, Steps<K>::Q> frag_perm(const T* row, int s, int lg) {
  using S = Steps<K>;
  static_assert(S::Q == 8, "two groups per step");
  Frag<T, 8> a;
  const T* p = row + 32 * s + 8 * lg;
  if constexpr (sizeof(T) == 2) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(p);
    a.w[0] = v.x; a.w[1] = v.y; a.w[2] = v.z; a.w[3] = v.w;
  } else {
    const u32x4 v0 = *reinterpret_cast<const u32x4*>(p), v1 = *reinterpret_cast<const u32x4*>(p + 4);
    a.w[0] = v0.x; a.w[1] = v0.y; a.w[2] = v0.z; a.w[3] = v0.w;
    a.w[4] = v1.x; a.w[5] = v1.y; a.w[6] = v1.z; a.w[7] = v1.w;
  }
  return a;
}

// ------------------------------------------------------------------ nodes

// Grid (ceil(n / 16), B): a block takes 16 nodes of graph blockIdx.y; wave w
// computes output features w D / 4 .. (w + 1) D / 4 - 1 (D / 64 tiles of 16)
// of all 16 rows. Each product's weight matrix is staged whole in LDS (the next one
// is loaded into registers while the current product and its layer norm
// run), and so is the product's input (O, then X1, then the hidden layer,
// rounded to T); layer-norm statistics combine over the waves through LDS.
// Writes X2 and the block's sums of X2 over its real nodes (part_x).
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void blk_node_kernel(BlockArgs k) {
  // FW features (TPW tiles of 16) per wave
  constexpr int EPC = 16 / (int)sizeof(T), LD = D + EPC, TPW = D / 64, FW = D / 4;
  static_assert(D % 64 == 0, "four waves of whole tiles");
  __shared__ __align__(16) T w_s[D][LD];
  __shared__ __align__(16) T in_s[16][LD];
  __shared__ float red_s[2][kWaves][16];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, li = l & 15, lg = l >> 4;
  const int b = blockIdx.y, n = k.n, i = blockIdx.x * 16 + li;
  const bool inr = i < n;
  const size_t row = (size_t)b * n + (inr ? i : 0);
  auto par = [&](int q) { return static_cast<const T*>(k.p[q]); };
  const size_t row0 = (size_t)b * n + blockIdx.x * 16;  // the block's first node row
  const int nrows = n - (int)blockIdx.x * 16 < 16 ? n - (int)blockIdx.x * 16 : 16;
  // the block's 16 rows of O (rows past n are clamped to the first row)
  auto load_rows = [&](Pieces<T, 16, D>& pc, const T* base) {
#pragma unroll
    for (int e = 0; e < Pieces<T, 16, D>::PER; ++e) {
      const int q = tid + e * kThreads, r = q / (D / EPC), rr = r < nrows ? r : 0;
      pc.v[e] = *reinterpret_cast<const u32x4*>(base + (row0 + rr) * D + EPC * (q % (D / EPC)));
    }
  };
  Pieces<T, D, D> wp;
  Pieces<T, 16, D> ip;
  wp.load(par(kBW_o), tid);
  load_rows(ip, static_cast<const T*>(k.O));
  const bool real = inr && k.mask[row] != 0;
  float xr[4 * TPW];  // X, this wave's features of row li
#pragma unroll
  for (int t = 0; t < TPW; ++t) ld4f<T>(xr + 4 * t, static_cast<const T*>(k.X) + row * D + FW * w + 16 * t + 4 * lg);
  wp.store(w_s, tid);
  ip.store(in_s, tid);
  __syncthreads();
  wp.load(par(kBW_x1), tid);  // in flight during the first product and its layer norm

  // out[4 TPW] = this wave's features of W in + bias, W and in from LDS
  auto gemm = [&](float* out, int bias_q) {
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const int o0 = FW * w + 16 * t;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s2 = 0; s2 < Steps<D>::NS; ++s2)
        acc = mma(acc, frag_at<T, D>(&w_s[o0 + li][0], s2, lg), frag_at<T, D>(&in_s[li][0], s2, lg));
      float bv[4];
      ld4f<T>(bv, par(bias_q) + o0 + 4 * lg);
#pragma unroll
      for (int r = 0; r < 4; ++r) out[4 * t + r] = acc[r] + bv[r];
    }
  };
  // layer norm over all D features of row li (this wave holds 4 TPW of them)
  auto ln = [&](float* v, int gq, int bq) {
    float sm = 0.f;
#pragma unroll
    for (int q = 0; q < 4 * TPW; ++q) sm += v[q];
    sm = lg_sum(sm);
    if (lg == 0) red_s[0][w][li] = sm;
    __syncthreads();
    const float mean = (red_s[0][0][li] + red_s[0][1][li] + red_s[0][2][li] + red_s[0][3][li]) * (1.f / D);
    float sq = 0.f;
#pragma unroll
    for (int q = 0; q < 4 * TPW; ++q) {
      v[q] -= mean;
      sq += v[q] * v[q];
    }
    sq = lg_sum(sq);
    if (lg == 0) red_s[1][w][li] = sq;
    __syncthreads();
    const float inv =
        1.f / sqrtf((red_s[1][0][li] + red_s[1][1][li] + red_s[1][2][li] + red_s[1][3][li]) * (1.f / D) + kLnEps);
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      float gv[4], bv[4];
      ld4f<T>(gv, par(gq) + FW * w + 16 * t + 4 * lg);
      ld4f<T>(bv, par(bq) + FW * w + 16 * t + 4 * lg);
#pragma unroll
      for (int r = 0; r < 4; ++r) v[4 * t + r] = v[4 * t + r] * inv * gv[r] + bv[r];
    }
  };
  // this wave's features of a row-layout vector into in_s (rounded to T)
  auto put_row = [&](const float* v) {
#pragma unroll
    for (int t = 0; t < TPW; ++t) st4f<T>(&in_s[li][FW * w + 16 * t + 4 * lg], v + 4 * t);
  };

  float x1[4 * TPW], z[4 * TPW];
  gemm(z, kBb_o);
#pragma unroll
  for (int q = 0; q < 4 * TPW; ++q) x1[q] = z[q] + xr[q];
  ln(x1, kBln_x1_g, kBln_x1_b);  // its barriers also end every wave's reads of w_s and in_s
  put_row(x1);
  wp.store(w_s, tid);
  __syncthreads();
  wp.load(par(kBW_x2), tid);
  gemm(z, kBb_x1);
#pragma unroll
  for (int q = 0; q < 4 * TPW; ++q) z[q] = fmaxf(z[q], 0.f);
  __syncthreads();  // every wave is done with w_s and in_s
  put_row(z);
  wp.store(w_s, tid);
  __syncthreads();
  gemm(z, kBb_x2);
#pragma unroll
  for (int q = 0; q < 4 * TPW; ++q) z[q] += x1[q];
  ln(z, kBln_x2_g, kBln_x2_b);
#pragma unroll
  for (int q = 0; q < 4 * TPW; ++q) z[q] = real ? z[q] : 0.f;
  if (inr) {
#pragma unroll
    for (int t = 0; t < TPW; ++t) st4f<T>(static_cast<T*>(k.X_out) + row * D + FW * w + 16 * t + 4 * lg, z + 4 * t);
  }
  // sums over the 16 rows (lanes li of a lane group) of the block's real nodes
#pragma unroll
  for (int q = 0; q < 4 * TPW; ++q) z[q] = row16_sum(z[q]);
  if (li == 0) {
    float* part = k.part_x + ((size_t)b * gridDim.x + blockIdx.x) * D;
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) part[FW * w + 16 * t + 4 * lg + r] = z[4 * t + r];
  }
}

// ------------------------------------------------------------------ edges

// Grid (EX, B), kEdgeWaves waves per block: the edge tokens (i, j) of graph
// blockIdx.y in tiles of 16; wave slot blockIdx.x * kEdgeWaves + w takes
// tiles slot, slot + kEdgeWaves EX, ... . Weights,
// biases and layer-norm parameters are staged in LDS once per block; the
// next tile's E' and mask bytes are loaded (raw, into the other of two
// register sets) while the current tile is computed. E2 is written over E'
// in place (each lane reads its token's row before writing it). Also the
// block's sums of E2 over its real pairs (part_e).
template <typename T, int DE>
__global__ __launch_bounds__(kEdgeWaves * 64) void blk_edge_kernel(BlockArgs k) {
  constexpr int FE = 2 * DE, EPC = 16 / (int)sizeof(T), NT = kEdgeWaves * 64;
  constexpr bool kPerm1 = Steps<DE>::Q == 8;
  __shared__ __align__(16) T w1_s[FE][DE + EPC];
  __shared__ __align__(16) T w2_s[DE][FE + EPC];
  __shared__ float pv_s[6][FE];  // b_e1, b_e2, ln_e1 g / b, ln_e2 g / b
  __shared__ float sum_s[kEdgeWaves][DE];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, li = l & 15, lg = l >> 4;
  const int b = blockIdx.y, n = k.n;
  auto par = [&](int q) { return static_cast<const T*>(k.p[q]); };
  T* Eio = static_cast<T*>(k.E_io);
  const int ntok = n * n, ntile = (ntok + 15) / 16;
  constexpr int DW = 4 * (int)sizeof(T) / 4;
  struct Raw {
    uint32_t e[DE / 16][DW];  // groups 16 t + 4 lg .. + 3 of the token's row
    uint8_t mi, mj;
  };
  auto tok = [&](int tile, int& i, int& j) {
    const int tk = 16 * tile + li, tc = tk < ntok ? tk : 0;
    i = tc / n;
    j = tc % n;
    return tk < ntok;
  };
  auto load = [&](int tile, Raw& r) {
    int i, j;
    tok(tile < ntile ? tile : 0, i, j);
    const T* rowp = Eio + (((size_t)b * n + i) * n + j) * DE;
#pragma unroll
    for (int t = 0; t < DE / 16; ++t) ld4w<T>(r.e[t], rowp + 16 * t + 4 * lg);
    r.mi = k.mask[(size_t)b * n + i];
    r.mj = k.mask[(size_t)b * n + j];
  };
  const int stride = gridDim.x * kEdgeWaves;
  Raw r0, r1;
  int tile = blockIdx.x * kEdgeWaves + w;
  if (tile < ntile) load(tile, r0);  // the first tile is in flight during the staging
  {
    // W_e1 keeps the plain layout when its contraction (DE = 16) is one group;
    // otherwise both are staged with the fragment-contiguous column order
    using P1 = typename std::conditional<kPerm1, PermStage<T, FE, DE, NT>, Pieces<T, FE, DE, NT>>::type;
    P1 p1;
    PermStage<T, DE, FE, NT> p2;
    p1.load(par(kBW_e1), tid);
    p2.load(par(kBW_e2), tid);
    const int pq[6] = {kBb_e1, kBb_e2, kBln_e1_g, kBln_e1_b, kBln_e2_g, kBln_e2_b};
    for (int q = tid; q < 6 * FE; q += NT) {
      const int v = q / FE, c = q % FE;
      if (v == 0 || c < DE) pv_s[v][c] = Num<T>::ld(par(pq[v]) + c);
    }
    p1.store(w1_s, tid);
    p2.store(w2_s, tid);
  }
  __syncthreads();
  // layer norm of this lane's DE / 4 features of its token (gain row gq, shift row bq of pv_s)
  auto lnv = [&](float* v, int gq, int bq) {
    float sm = 0.f;
#pragma unroll
    for (int q = 0; q < DE / 4; ++q) sm += v[q];
    const float mean = lg_sum(sm) * (1.f / DE);
    float sq = 0.f;
#pragma unroll
    for (int q = 0; q < DE / 4; ++q) {
      v[q] -= mean;
      sq += v[q] * v[q];
    }
    const float inv = 1.f / sqrtf(lg_sum(sq) * (1.f / DE) + kLnEps);
#pragma unroll
    for (int t = 0; t < DE / 16; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int c = 16 * t + 4 * lg + r;
        v[4 * t + r] = v[4 * t + r] * inv * pv_s[gq][c] + pv_s[bq][c];
      }
  };
  float esum[DE / 4];
#pragma unroll
  for (int q = 0; q < DE / 4; ++q) esum[q] = 0.f;
  auto step = [&](int tile, const Raw& cur, Raw& nxt) {
    load(tile + gridDim.x * kEdgeWaves, nxt);
    __builtin_amdgcn_sched_barrier(0);  // the next tile's loads stay ahead of this tile's work
    int i, j;
    const bool valid = tok(tile, i, j);
    const bool real = valid && cur.mi != 0 && cur.mj != 0;
    float e1[DE / 4], h[FE / 4], z[DE / 4];
#pragma unroll
    for (int t = 0; t < DE / 16; ++t) {
      if constexpr (sizeof(T) == 2) {
        e1[4 * t] = __uint_as_float(cur.e[t][0] << 16); e1[4 * t + 1] = __uint_as_float(cur.e[t][0] & 0xffff0000u);
        e1[4 * t + 2] = __uint_as_float(cur.e[t][1] << 16); e1[4 * t + 3] = __uint_as_float(cur.e[t][1] & 0xffff0000u);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) e1[4 * t + r] = __uint_as_float(cur.e[t][r]);
      }
    }
    lnv(e1, 2, 3);
    {
      RowIn<T, DE> in;
      in.set(e1);
#pragma unroll
      for (int to = 0; to < FE / 16; ++to) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s2 = 0; s2 < Steps<DE>::NS; ++s2) {
          if constexpr (kPerm1) acc = mma(acc, frag_perm<T, DE>(&w1_s[16 * to + li][0], s2, lg), in.f[s2]);
          else acc = mma(acc, frag_at<T, DE>(&w1_s[16 * to + li][0], s2, lg), in.f[s2]);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) h[4 * to + r] = fmaxf(acc[r] + pv_s[0][16 * to + 4 * lg + r], 0.f);
      }
    }
    {
      RowIn<T, FE> in;
      in.set(h);
#pragma unroll
      for (int to = 0; to < DE / 16; ++to) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s2 = 0; s2 < Steps<FE>::NS; ++s2) acc = mma(acc, frag_perm<T, FE>(&w2_s[16 * to + li][0], s2, lg), in.f[s2]);
#pragma unroll
        for (int r = 0; r < 4; ++r) z[4 * to + r] = acc[r] + pv_s[1][16 * to + 4 * lg + r] + e1[4 * to + r];
      }
    }
    lnv(z, 4, 5);
#pragma unroll
    for (int q = 0; q < DE / 4; ++q) {
      z[q] = real ? z[q] : 0.f;
      esum[q] += z[q];
    }
    if (valid) {
      T* rowp = Eio + (((size_t)b * n + i) * n + j) * DE;
#pragma unroll
      for (int t = 0; t < DE / 16; ++t) st4f<T>(rowp + 16 * t + 4 * lg, z + 4 * t);
    }
  };
  for (; tile < ntile; tile += 2 * stride) {
    step(tile, r0, r1);
    if (tile + stride >= ntile) break;
    step(tile + stride, r1, r0);
  }
  // sums over the 16 tokens (lanes li), then over the waves
#pragma unroll
  for (int q = 0; q < DE / 4; ++q) esum[q] = row16_sum(esum[q]);
  if (li == 0) {
#pragma unroll
    for (int t = 0; t < DE / 16; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) sum_s[w][16 * t + 4 * lg + r] = esum[4 * t + r];
  }
  __syncthreads();
  float* part = k.part_e + ((size_t)b * gridDim.x + blockIdx.x) * DE;
  for (int f = tid; f < DE; f += NT) {
    float t = 0.f;
#pragma unroll
    for (int q = 0; q < kEdgeWaves; ++q) t += sum_s[q][f];
    part[f] = t;
  }
}

// ------------------------------------------------------------------ y

// Weights of one output row, lane l taking inputs l, l + 64, ... (raw words;
// lanes past LEN load element 0 and later count as 0).
template <typename T, int LEN>
struct RowW {
  static constexpr int U = (LEN + 63) / 64;
  uint32_t w[U];
  __device__ __forceinline__ void load(const T* row, int l) {
#pragma unroll
    for (int u = 0; u < U; ++u) w[u] = Num<T>::ldraw(row + (l + 64 * u < LEN ? l + 64 * u : 0));
  }
  // this lane's part of the row times v (v in LDS)
  __device__ __forceinline__ float dot(const float* v, int l) const {
    float s = 0.f;
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (LEN % 64 == 0 || l + 64 * u < LEN) s += Num<T>::fromraw(w[u]) * v[l + 64 * u];
    return s;
  }
};


// One block per graph: the means from the partial sums, then the y path in
// float32. Wave w computes outputs o = w, w + 4, ...; its lanes read
// consecutive weights of the output's row (one cache line per load) and sum
// over the wave. Every weight and parameter is loaded at the start, so the
// chain of products and norms that follows waits on no memory.
template <typename T, int D, int DE, int DY>
__global__ __launch_bounds__(kThreads) void blk_y_kernel(BlockArgs k) {
  constexpr int OPW = DY / kWaves;  // outputs per wave
  static_assert(DY % kWaves == 0 && DY <= kThreads && D <= kThreads && DE <= kThreads, "one feature per thread");
  static_assert(kThreads % D == 0 && kThreads % DE == 0, "partial-sum groups");
  __shared__ float xbar[D], ebar[DE], tail_x[kThreads], tail_e[kThreads];
  __shared__ float yv[DY], y1[DY], hy[DY], red4[2][kWaves];
  __shared__ int cnt;
  const int tid = threadIdx.x, b = blockIdx.x, n = k.n, w = tid >> 6, l = tid & 63;
  auto par = [&](int q) { return static_cast<const T*>(k.p[q]); };
  // First-phase loads (mask bytes, y, the first partial sums) are issued
  // before the weights: loads complete in issue order, so waiting for them
  // does not wait for the weights, which arrive during the sums.
  constexpr int NMK = 4, NPB = 16;  // mask bytes and partials per thread held in registers
  uint8_t mk[NMK];
#pragma unroll
  for (int q = 0; q < NMK; ++q) {
    const int i = tid + q * kThreads;
    mk[q] = k.mask[(size_t)b * n + (i < n ? i : 0)];
  }
  const int cc = tid < DY ? tid : 0;  // feature of the norm and bias steps
  const float yr = Num<T>::ld(static_cast<const T*>(k.y) + (size_t)b * DY + cc);
  const int fx = tid < D ? tid : 0, fe = tid < DE ? tid : 0;
  float px[NPB], pe[NPB];
#pragma unroll
  for (int q = 0; q < NPB; ++q) {
    px[q] = k.part_x[((size_t)b * k.nxb + (q < k.nxb ? q : 0)) * D + fx];
    pe[q] = k.part_e[((size_t)b * k.exb + (q < k.exb ? q : 0)) * DE + fe];
  }
  __builtin_amdgcn_sched_barrier(0);
  RowW<T, D> wyx[OPW];
  RowW<T, DE> wye[OPW];
  RowW<T, DY> wyy[OPW], wy1[OPW], wy2[OPW];
#pragma unroll
  for (int m = 0; m < OPW; ++m) {
    const size_t o = w + kWaves * m;
    wyx[m].load(par(kBW_yx) + o * D, l);
    wye[m].load(par(kBW_ye) + o * DE, l);
    wyy[m].load(par(kBW_yy) + o * DY, l);
    wy1[m].load(par(kBW_y1) + o * DY, l);
    wy2[m].load(par(kBW_y2) + o * DY, l);
  }
  const uint32_t pb[3] = {Num<T>::ldraw(par(kBb_yo) + cc), Num<T>::ldraw(par(kBb_y1) + cc),
                          Num<T>::ldraw(par(kBb_y2) + cc)};
  const uint32_t pl[4] = {Num<T>::ldraw(par(kBln_y1_g) + cc), Num<T>::ldraw(par(kBln_y1_b) + cc),
                          Num<T>::ldraw(par(kBln_y2_g) + cc), Num<T>::ldraw(par(kBln_y2_b) + cc)};
  __builtin_amdgcn_sched_barrier(0);
  if (tid == 0) cnt = 0;
  __syncthreads();
  int c0 = 0;
#pragma unroll
  for (int q = 0; q < NMK; ++q) c0 += (tid + q * kThreads < n && mk[q] != 0) ? 1 : 0;
  for (int i = tid + NMK * kThreads; i < n; i += kThreads) c0 += k.mask[(size_t)b * n + i] != 0;
  atomicAdd(&cnt, c0);
  if (tid < DY) yv[tid] = yr;
  // Partial sums past the first NPB (large graphs have up to 256 edge blocks):
  // every thread takes feature tid % F of partials NPB + tid / F, stepping by
  // kThreads / F, with U independent loads in flight, instead of one thread
  // per feature walking a chain of dependent loads.
  auto tail = [&](const float* part, int cnt, int F) {
    constexpr int U = 16;
    const int G = kThreads / F, f = tid % F;
    float acc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) acc[u] = 0.f;
    int q = NPB + tid / F;
    for (; q + (U - 1) * G < cnt; q += U * G) {
      float v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = part[(size_t)(q + u * G) * F + f];
#pragma unroll
      for (int u = 0; u < U; ++u) acc[u] += v[u];
    }
    for (; q < cnt; q += G) acc[0] += part[(size_t)q * F + f];
    float t = 0.f;
#pragma unroll
    for (int u = 0; u < U; ++u) t += acc[u];
    return t;
  };
  tail_x[tid] = tail(k.part_x + (size_t)b * k.nxb * D, k.nxb, D);
  tail_e[tid] = tail(k.part_e + (size_t)b * k.exb * DE, k.exb, DE);
  __syncthreads();
  const float nr = (float)cnt;
  if (tid < D) {
    float sx = 0.f;
#pragma unroll
    for (int q = 0; q < NPB; ++q) sx += q < k.nxb ? px[q] : 0.f;
    for (int g = 0; g < kThreads / D; ++g) sx += tail_x[g * D + tid];
    xbar[tid] = sx / fmaxf(nr, 1.f);
  }
  if (tid < DE) {
    float se = 0.f;
#pragma unroll
    for (int q = 0; q < NPB; ++q) se += q < k.exb ? pe[q] : 0.f;
    for (int g = 0; g < kThreads / DE; ++g) se += tail_e[g * DE + tid];
    ebar[tid] = se / fmaxf(nr * nr, 1.f);
  }
  __syncthreads();
  // sum of x over all threads of the block (every thread gets it)
  auto block_sum = [&](float x, int slot) {
    x = wave64_sum(x);
    if (l == 0) red4[slot][w] = x;
    __syncthreads();
    return red4[slot][0] + red4[slot][1] + red4[slot][2] + red4[slot][3];
  };
  auto block_ln = [&](float* v, uint32_t g, uint32_t bb) {
    const float x = tid < DY ? v[cc] : 0.f;
    const float mean = block_sum(x, 0) * (1.f / DY);
    const float dv = tid < DY ? x - mean : 0.f;
    const float inv = 1.f / sqrtf(block_sum(dv * dv, 1) * (1.f / DY) + kLnEps);
    if (tid < DY) v[tid] = dv * inv * Num<T>::fromraw(g) + Num<T>::fromraw(bb);
    __syncthreads();
  };
#pragma unroll
  for (int m = 0; m < OPW; ++m) {
    const float s = wave64_sum(wyx[m].dot(xbar, l) + wye[m].dot(ebar, l) + wyy[m].dot(yv, l));
    if (l == 0) y1[w + kWaves * m] = s;
  }
  __syncthreads();
  if (tid < DY) y1[tid] += yv[tid] + Num<T>::fromraw(pb[0]);
  __syncthreads();
  block_ln(y1, pl[0], pl[1]);
#pragma unroll
  for (int m = 0; m < OPW; ++m) {
    const float s = wave64_sum(wy1[m].dot(y1, l));
    if (l == 0) hy[w + kWaves * m] = s;
  }
  __syncthreads();
  if (tid < DY) hy[tid] = fmaxf(hy[tid] + Num<T>::fromraw(pb[1]), 0.f);
  __syncthreads();
#pragma unroll
  for (int m = 0; m < OPW; ++m) {
    const float s = wave64_sum(wy2[m].dot(hy, l));
    if (l == 0) yv[w + kWaves * m] = s;  // y is no longer needed
  }
  __syncthreads();
  if (tid < DY) yv[tid] += y1[tid] + Num<T>::fromraw(pb[2]);
  __syncthreads();
  block_ln(yv, pl[2], pl[3]);
  if (tid < DY) Num<T>::st(static_cast<T*>(k.y_out) + (size_t)b * DY + tid, yv[tid]);
}

template <typename T, int D, int DE, int DY>
hipError_t block_shape(const BlockArgs& k, hipStream_t s) {
  hipLaunchKernelGGL((blk_node_kernel<T, D>), dim3(k.nxb, k.B), dim3(kThreads), 0, s, k);
  hipLaunchKernelGGL((blk_edge_kernel<T, DE>), dim3(k.exb, k.B), dim3(kEdgeWaves * 64), 0, s, k);
  hipLaunchKernelGGL((blk_y_kernel<T, D, DE, DY>), dim3(k.B), dim3(kThreads), 0, s, k);
  return hipGetLastError();
}

}  // namespace

bool block_supported(int dtype, int d, int de, int dy) {
  return (dtype == 1 && d == 256 && de == 64 && dy == 64) || (d == 64 && de == 16 && dy == 16);
}

hipError_t launch_block(const BlockArgs& k, int dtype, int d, int de, hipStream_t s) {
  if (dtype == 1 && d == 256 && de == 64 && k.dy == 64) return block_shape<bf16_t, 256, 64, 64>(k, s);
  if (dtype == 1 && d == 64 && de == 16 && k.dy == 16) return block_shape<bf16_t, 64, 16, 16>(k, s);
  if (dtype == 0 && d == 64 && de == 16 && k.dy == 16) return block_shape<float, 64, 16, 16>(k, s);
  return hipErrorInvalidValue;
}

}  // namespace ea
