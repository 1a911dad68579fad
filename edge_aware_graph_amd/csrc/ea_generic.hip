// Generic gfx950 path of the edge-aware attention layer: every shape the
// boundary accepts (head width dh in {16, 32, 64}, edge width de a multiple
// of 16, 2H <= 32, any n), with the sizes as runtime values.
//
// It computes the same layer as the tuned kernels ("Efficient Edge-aware
// Attention Network for Graph Generation", ai-frontier-tracker digest,
// full-text summary: scaled dot-product scores, head-wise FiLM of the score
// from the edge and the global feature, graph mask, normalized softmax,
// A [V | I] giving O and A, residual edge update E' = E + W_e A + b_e; large
// graphs in two passes) with the same bfloat16 rounding points: Q, K, V
// rounded after the projection, A rounded before it is stored, multiplied
// with V and used in the update.
//
// One block per (graph, query row) walks the row's keys in chunks of 256,
// one key per thread, twice: the first walk only finds the row's softmax
// statistics (running max and sum per head, online), the second recomputes
// the logits, forms the normalized A, accumulates O (threads over output
// columns) and writes E'. That is the pages' two-pass scheme applied inside
// one block, so a row of any length fits; E of the row is read twice.
// Plain VALU arithmetic in float32: this path trades speed for generality.
#include "ea_device.h"

#include <math.h>

namespace ea {
namespace {

constexpr int kGenThreads = 256;
constexpr int kGenChunk = 256;  // keys per chunk (one per thread)
constexpr int kMaxHeads = 16;   // 2H <= 32
constexpr int kMaxD = 1024;     // H dh <= 16 * 64

// Q | K | V = X W^T + b per real row, zeros for padded rows and the slots
// [n, NP); Q, K [B, H, NP, dh], V^T [B, H, dh, NP] (the tuned kernels'
// workspace layout). One thread per output element.
template <typename T>
__global__ __launch_bounds__(kGenThreads) void gen_qkv_kernel(LayerArgs a) {
  const int d = a.d, dh = a.dh, H = a.H, NP = a.NP, n = a.n;
  const size_t total = (size_t)a.B * NP * 3 * d;
  for (size_t idx = (size_t)blockIdx.x * kGenThreads + threadIdx.x; idx < total;
       idx += (size_t)gridDim.x * kGenThreads) {
    const int f = (int)(idx % (3 * d));
    const size_t row = idx / (3 * d);
    const int b = (int)(row / NP), i = (int)(row % NP);
    const int which = f / d, fl = f % d, h = fl / dh, t = fl % dh;
    const bool real = i < n && a.mask[(size_t)b * n + i] != 0;
    float acc = 0.f;
    if (real) {
      const T* x = static_cast<const T*>(a.X) + ((size_t)b * n + i) * d;
      const T* w = static_cast<const T*>(which == 0 ? a.w_q : which == 1 ? a.w_k : a.w_v) + (size_t)fl * d;
      for (int c = 0; c < d; ++c) acc = fmaf(Num<T>::ld(x + c), Num<T>::ld(w + c), acc);
      const void* bias = which == 0 ? a.b_q : which == 1 ? a.b_k : a.b_v;
      if (bias) acc += Num<T>::ld(static_cast<const T*>(bias) + fl);
    }
    const float v = real ? acc : 0.f;
    if (which == 2)
      Num<T>::st(static_cast<T*>(a.Vt) + (((size_t)b * H + h) * dh + t) * NP + i, v);
    else
      Num<T>::st(static_cast<T*>(which == 0 ? a.Qw : a.Kw) + (((size_t)b * H + h) * NP + i) * dh + t, v);
  }
}

// gamma_y = 1 + W_ymul y + b_ymul, beta_y = W_yadd y + b_yadd per graph;
// (1, 0) without score modulation. One thread per (graph, coefficient).
template <typename T>
__global__ __launch_bounds__(kGenThreads) void gen_gy_kernel(LayerArgs a) {
  const int H = a.H;
  const int idx = blockIdx.x * kGenThreads + threadIdx.x;
  if (idx >= a.B * 2 * H) return;
  const int b = idx / (2 * H), o = idx % (2 * H), h = o % H;
  if (a.variant & kNoScoreMod) {
    a.gy[idx] = o < H ? 1.f : 0.f;
    return;
  }
  const T* w = static_cast<const T*>(o < H ? a.w_ymul : a.w_yadd) + (size_t)h * a.dy;
  const T* y = static_cast<const T*>(a.y) + (size_t)b * a.dy;
  float acc = 0.f;
  for (int c = 0; c < a.dy; ++c) acc = fmaf(Num<T>::ld(y + c), Num<T>::ld(w + c), acc);
  const void* bias = o < H ? a.b_ymul : a.b_yadd;
  if (bias) acc += Num<T>::ld(static_cast<const T*>(bias) + h);
  a.gy[idx] = o < H ? 1.f + acc : acc;
}

// Max / sum over the 16 lanes of a lane group; every lane gets the same bits
// (each butterfly step adds the same two values in both partner lanes).
__device__ __forceinline__ float group16_max(float v) {
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 16));
  return v;
}
__device__ __forceinline__ float group16_sum(float v) {
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) v += __shfl_xor(v, m, 16);
  return v;
}

struct GenShared {
  float q[kMaxD];                       // the query row, all heads
  float p[kGenChunk][kMaxHeads + 1];    // logits, then A, of the chunk's keys
  float gy[2 * kMaxHeads];
  float M[kMaxHeads], L[kMaxHeads];     // row statistics per head
};

// Masked logits u[h] of pair (i, j) (-inf unless both nodes are real).
template <typename T>
__device__ __forceinline__ void gen_logits(const LayerArgs& a, const GenShared& sh, int b, int i, int j, bool valid,
                                           float (&u)[kMaxHeads]) {
  const int H = a.H, dh = a.dh, de = a.de, NP = a.NP;
#pragma unroll
  for (int h = 0; h < kMaxHeads; ++h) u[h] = kNegInf;
  if (!valid) return;
  float ge[kMaxHeads], be[kMaxHeads];
  const bool film = (a.variant & (kLightEdge | kNoScoreMod)) == 0;
#pragma unroll
  for (int h = 0; h < kMaxHeads; ++h) {
    ge[h] = 1.f;
    be[h] = 0.f;
    if (film && h < H) {
      if (a.b_emul) ge[h] += Num<T>::ld(static_cast<const T*>(a.b_emul) + h);
      if (a.b_eadd) be[h] += Num<T>::ld(static_cast<const T*>(a.b_eadd) + h);
    }
  }
  if (film) {
    const T* e = static_cast<const T*>(a.E) + (((size_t)b * a.n + i) * a.n + j) * de;
    const T* wm = static_cast<const T*>(a.w_emul);
    const T* wa = static_cast<const T*>(a.w_eadd);
    for (int c = 0; c < de; ++c) {
      const float ev = Num<T>::ld(e + c);
#pragma unroll
      for (int h = 0; h < kMaxHeads; ++h) {
        if (h < H) {
          ge[h] = fmaf(ev, Num<T>::ld(wm + (size_t)h * de + c), ge[h]);
          be[h] = fmaf(ev, Num<T>::ld(wa + (size_t)h * de + c), be[h]);
        }
      }
    }
  }
  const T* K = static_cast<const T*>(a.Kw);
#pragma unroll
  for (int h = 0; h < kMaxHeads; ++h) {
    if (h >= H) continue;
    const T* k = K + (((size_t)b * H + h) * NP + j) * dh;
    float s = 0.f;
    for (int t = 0; t < dh; ++t) s = fmaf(sh.q[h * dh + t], Num<T>::ld(k + t), s);
    s *= a.scale;
    u[h] = (s * ge[h] + be[h]) * sh.gy[h] + sh.gy[H + h];
  }
}

// One block per (query row i, graph b); see the file comment.
template <typename T, int MODE>
__global__ __launch_bounds__(kGenThreads) void gen_row_kernel(LayerArgs a, int two_pass) {
  __shared__ GenShared sh;
  const int i = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int n = a.n, H = a.H, dh = a.dh, de = a.de, d = a.d, NP = a.NP;
  const uint8_t* mask_b = a.mask + (size_t)b * n;
  const bool mi = mask_b[i] != 0;
  const bool unnorm = (a.variant & kUnnormalized) != 0;
  T* Eout = static_cast<T*>(a.E_out);

  if (!mi) {  // padded query: zero outputs only
    for (int j = tid; j < n; j += kGenThreads) {
      if (MODE == kGenLogits) {
        for (int h = 0; h < H; ++h) a.U[(((size_t)b * H + h) * n + i) * n + j] = kNegInf;
      }
      if ((MODE == kGenForward || MODE == kGenLayer) && !two_pass) {
        for (int h = 0; h < H; ++h) Num<T>::st(static_cast<T*>(a.A) + (((size_t)b * H + h) * n + i) * n + j, 0.f);
      }
      if (MODE == kGenLayer || MODE == kGenUpdate) {
        T* row = Eout + (((size_t)b * n + i) * n + j) * de;
        for (int c = 0; c < de; ++c) Num<T>::st(row + c, 0.f);
      }
    }
    if (MODE == kGenForward || MODE == kGenLayer) {
      for (int c = tid; c < d; c += kGenThreads) Num<T>::st(static_cast<T*>(a.O) + ((size_t)b * n + i) * d + c, 0.f);
      if (MODE == kGenForward && two_pass && tid < H) a.lse[((size_t)b * H + tid) * NP + i] = kNegInf;
    }
    return;
  }

  const bool need_stats = MODE == kGenForward || MODE == kGenLayer;
  // the logits are recomputed unless a single-pass update reads the stored A
  const bool need_u = MODE == kGenLogits || need_stats || (MODE == kGenUpdate && (two_pass || unnorm));
  if (need_u) {  // query row and global FiLM coefficients (the workspace is only read then)
    for (int c = tid; c < d; c += kGenThreads) {
      const int h = c / dh, t = c % dh;
      sh.q[c] = Num<T>::ld(static_cast<const T*>(a.Qw) + (((size_t)b * H + h) * NP + i) * dh + t);
    }
    if (tid < 2 * H) sh.gy[tid] = a.gy[(size_t)b * 2 * H + tid];
    __syncthreads();
  }

  const int hh = tid >> 4, part = tid & 15;  // statistics: 16 threads per head
  if (need_stats) {
    float Mrun = kNegInf, Lrun = 0.f;
    for (int j0 = 0; j0 < n; j0 += kGenChunk) {
      const int j = j0 + tid, cnt = min(kGenChunk, n - j0);
      const bool valid = j < n && mask_b[j] != 0;
      float u[kMaxHeads];
      gen_logits<T>(a, sh, b, i, j, valid, u);
      if (tid < cnt)
        for (int h = 0; h < H; ++h) sh.p[tid][h] = u[h];
      __syncthreads();
      if (hh < H) {
        float m = kNegInf;
        for (int k = part; k < cnt; k += 16) m = fmaxf(m, sh.p[k][hh]);
        m = group16_max(m);
        const float Mn = fmaxf(Mrun, m);
        float s = 0.f;
        if (Mn != kNegInf)
          for (int k = part; k < cnt; k += 16) {
            const float v = sh.p[k][hh];
            s += v == kNegInf ? 0.f : expf(v - Mn);
          }
        s = group16_sum(s);
        Lrun = (Mrun == kNegInf ? 0.f : Lrun * expf(Mrun - Mn)) + s;
        Mrun = Mn;
      }
      __syncthreads();
    }
    if (hh < H && part == 0) {
      sh.M[hh] = Mrun;
      sh.L[hh] = Lrun;
    }
    __syncthreads();
  } else if (MODE == kGenUpdate && two_pass) {
    if (tid < H) sh.M[tid] = a.lse[((size_t)b * H + tid) * NP + i];
    __syncthreads();
  }

  float oacc[kMaxD / kGenThreads];
#pragma unroll
  for (int q = 0; q < kMaxD / kGenThreads; ++q) oacc[q] = 0.f;
  const T* W_e = static_cast<const T*>(a.w_e);
  const T* b_e = static_cast<const T*>(a.b_e);

  for (int j0 = 0; j0 < n; j0 += kGenChunk) {
    const int j = j0 + tid, cnt = min(kGenChunk, n - j0);
    const bool inb = j < n;
    const bool valid = inb && mask_b[j] != 0;
    float u[kMaxHeads];
    if (need_u) gen_logits<T>(a, sh, b, i, j, valid, u);
    else
#pragma unroll
      for (int h = 0; h < kMaxHeads; ++h) u[h] = 0.f;
    if (MODE == kGenLogits) {
      if (inb)
        for (int h = 0; h < H; ++h) a.U[(((size_t)b * H + h) * n + i) * n + j] = u[h];
      continue;
    }
    // A of this key for every head, rounded to the storage type
    float A[kMaxHeads];
#pragma unroll
    for (int h = 0; h < kMaxHeads; ++h) {
      float v = 0.f;
      if (h < H && valid) {
        if (need_stats) {
          v = sh.L[h] > 0.f ? expf(u[h] - sh.M[h]) / sh.L[h] : 0.f;
        } else if (two_pass) {
          v = sh.M[h] == kNegInf ? 0.f : expf(u[h] - sh.M[h]);
        } else if (!unnorm) {
          v = Num<T>::ld(static_cast<const T*>(a.A) + (((size_t)b * H + h) * n + i) * n + j);
        }
      }
      A[h] = Num<T>::rnd(v);
    }
    if (need_stats) {
      if (!two_pass && inb)
        for (int h = 0; h < H; ++h) Num<T>::st(static_cast<T*>(a.A) + (((size_t)b * H + h) * n + i) * n + j, A[h]);
      if (tid < cnt)
        for (int h = 0; h < H; ++h) sh.p[tid][h] = A[h];
    }
    if ((MODE == kGenLayer || MODE == kGenUpdate) && inb) {
      // residual edge update; the unnormalized variant takes u (0 at masked pairs)
      float op[kMaxHeads];
#pragma unroll
      for (int h = 0; h < kMaxHeads; ++h) op[h] = unnorm ? Num<T>::rnd(valid && h < H ? u[h] : 0.f) : A[h];
      T* row = Eout + (((size_t)b * n + i) * n + j) * de;
      const T* erow = static_cast<const T*>(a.E) + (((size_t)b * n + i) * n + j) * de;
      for (int c = 0; c < de; ++c) {
        float v = 0.f;
        if (valid) {
          v = Num<T>::ld(erow + c) + (b_e ? Num<T>::ld(b_e + c) : 0.f);
#pragma unroll
          for (int h = 0; h < kMaxHeads; ++h)
            if (h < H) v = fmaf(op[h], Num<T>::ld(W_e + (size_t)c * H + h), v);
        }
        Num<T>::st(row + c, v);
      }
    }
    if (need_stats) {
      __syncthreads();
      // O += A V over this chunk: threads over output columns c = h dh + t
#pragma unroll
      for (int q = 0; q < kMaxD / kGenThreads; ++q) {
        const int c = tid + q * kGenThreads;
        if (c < d) {
          const int h = c / dh, t = c % dh;
          const T* v = static_cast<const T*>(a.Vt) + (((size_t)b * H + h) * dh + t) * NP + j0;
          float s = oacc[q];
          for (int k = 0; k < cnt; ++k) s = fmaf(sh.p[k][h], Num<T>::ld(v + k), s);
          oacc[q] = s;
        }
      }
      __syncthreads();
    }
  }
  if (need_stats) {
#pragma unroll
    for (int q = 0; q < kMaxD / kGenThreads; ++q) {
      const int c = tid + q * kGenThreads;
      if (c < d) Num<T>::st(static_cast<T*>(a.O) + ((size_t)b * n + i) * d + c, oacc[q]);
    }
    if (MODE == kGenForward && two_pass && tid < H)
      a.lse[((size_t)b * H + tid) * NP + i] = sh.L[tid] > 0.f ? sh.M[tid] + logf(sh.L[tid]) : kNegInf;
  }
}

// A = softmax over the last axis of float32 logits (-inf = masked), a row
// without a finite logit gives 0; rounded to the storage type. One block per row.
template <typename T>
__global__ __launch_bounds__(kGenThreads) void gen_softmax_kernel(const float* U, T* A, int n) {
  __shared__ float red[kGenThreads / 64];
  const size_t row = (size_t)blockIdx.x + (size_t)blockIdx.y * gridDim.x;
  const float* u = U + row * n;
  T* out = A + row * n;
  const int tid = threadIdx.x, w = tid >> 6;
  float m = kNegInf;
  for (int j = tid; j < n; j += kGenThreads) m = fmaxf(m, u[j]);
  m = fmaxf(m, __shfl_xor(m, 32));
  m = fmaxf(m, __shfl_xor(m, 16));
  m = group16_max(m);  // all 64 lanes
  if ((tid & 63) == 0) red[w] = m;
  __syncthreads();
  float M = kNegInf;
  for (int k = 0; k < kGenThreads / 64; ++k) M = fmaxf(M, red[k]);
  __syncthreads();
  float s = 0.f;
  if (M != kNegInf)
    for (int j = tid; j < n; j += kGenThreads) s += u[j] == kNegInf ? 0.f : expf(u[j] - M);
  s += __shfl_xor(s, 32);
  s += __shfl_xor(s, 16);
  s = group16_sum(s);  // all 64 lanes
  if ((tid & 63) == 0) red[w] = s;
  __syncthreads();
  float L = 0.f;
  for (int k = 0; k < kGenThreads / 64; ++k) L += red[k];
  for (int j = tid; j < n; j += kGenThreads) {
    const float v = (L > 0.f && u[j] != kNegInf) ? expf(u[j] - M) / L : 0.f;
    Num<T>::st(out + j, v);
  }
}

template <typename T>
hipError_t gen_row_dispatch(const LayerArgs& a, int mode, int two_pass, hipStream_t s) {
  const dim3 grid(a.n, a.B);
  switch (mode) {
    case kGenForward: hipLaunchKernelGGL((gen_row_kernel<T, kGenForward>), grid, dim3(kGenThreads), 0, s, a, two_pass); break;
    case kGenLayer: hipLaunchKernelGGL((gen_row_kernel<T, kGenLayer>), grid, dim3(kGenThreads), 0, s, a, two_pass); break;
    case kGenUpdate: hipLaunchKernelGGL((gen_row_kernel<T, kGenUpdate>), grid, dim3(kGenThreads), 0, s, a, two_pass); break;
    case kGenLogits: hipLaunchKernelGGL((gen_row_kernel<T, kGenLogits>), grid, dim3(kGenThreads), 0, s, a, two_pass); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gen_qkv(const LayerArgs& a, int dtype, hipStream_t s) {
  const size_t total = (size_t)a.B * a.NP * 3 * a.d;
  const size_t want = (total + kGenThreads - 1) / kGenThreads;
  const unsigned blocks = (unsigned)(want < 65536 ? want : 65536);
  const unsigned gyb = (unsigned)((a.B * 2 * a.H + kGenThreads - 1) / kGenThreads);
  if (dtype == 1) {
    hipLaunchKernelGGL((gen_qkv_kernel<bf16_t>), dim3(blocks), dim3(kGenThreads), 0, s, a);
    hipLaunchKernelGGL((gen_gy_kernel<bf16_t>), dim3(gyb), dim3(kGenThreads), 0, s, a);
  } else {
    hipLaunchKernelGGL((gen_qkv_kernel<float>), dim3(blocks), dim3(kGenThreads), 0, s, a);
    hipLaunchKernelGGL((gen_gy_kernel<float>), dim3(gyb), dim3(kGenThreads), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_gen_row(const LayerArgs& a, int dtype, int mode, int two_pass, hipStream_t s) {
  return dtype == 1 ? gen_row_dispatch<bf16_t>(a, mode, two_pass, s) : gen_row_dispatch<float>(a, mode, two_pass, s);
}

hipError_t launch_gen_softmax(const float* U, void* A, long rows, int n, int dtype, hipStream_t s) {
  // rows = B H n < 2^31: split over a 2-D grid
  if (rows <= 0) return hipSuccess;
  const unsigned gx = (unsigned)(rows < 65536 ? rows : 65536);
  const unsigned gy = (unsigned)((rows + gx - 1) / gx);
  if ((long)gx * gy != rows) {
    // launch whole 65536-row slabs, then the rest
    const long slabs = rows / 65536, rest = rows % 65536;
    hipError_t e = launch_gen_softmax(U, A, slabs * 65536, n, dtype, s);
    if (e != hipSuccess) return e;
    const size_t es = dtype == 1 ? 2 : 4;
    return launch_gen_softmax(U + (size_t)slabs * 65536 * n, static_cast<char*>(A) + (size_t)slabs * 65536 * n * es,
                              rest, n, dtype, s);
  }
  if (dtype == 1)
    hipLaunchKernelGGL((gen_softmax_kernel<bf16_t>), dim3(gx, gy), dim3(kGenThreads), 0, s, U,
                       static_cast<bf16_t*>(A), n);
  else
    hipLaunchKernelGGL((gen_softmax_kernel<float>), dim3(gx, gy), dim3(kGenThreads), 0, s, U,
                       static_cast<float*>(A), n);
  return hipGetLastError();
}

}  // namespace ea
