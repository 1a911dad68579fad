// gfx950 (MI355X, CDNA4) kernels of the edge-aware attention layer.
//
// The layer follows "Efficient Edge-aware Attention Network for Graph
// Generation" (ai-frontier-tracker digest, full-text summary): scaled
// dot-product scores, head-wise FiLM of the edge features and of the global
// feature applied to the score, the graph mask, a normalized softmax, the
// A [V | I] product that returns the node aggregation and the attention map
// together, and a residual edge update from the attention map; large graphs
// take two passes.
//
// MFMA operand convention used by every contraction below. For a 16x16 output
// tile D = A (16 x K) * B (K x 16), lane l = 16*lg + li (li = l % 16,
// lg = l / 16) supplies row li of A and column li of B, restricted to the
// contiguous quarter [lg*K/4, (lg+1)*K/4) of the contraction; both operands
// use the same split, so any K is consumed by a chain of 16x16x32 bf16,
// 16x16x16 bf16 or 16x16x4 f32 MFMAs. The result leaves D[4*lg + r][li] in
// accumulator r of lane l.
//
// Score tiles are computed transposed, S^T = K Q^T, so lane (li, lg) holds
// the logits of query row i0 + li for the four keys j0 + 4*lg + r. That is
// exactly the B-operand layout of the next contraction O^T = V^T A^T (keys
// are the contraction), so the softmax output feeds the MFMA without moving.
#include "ea_internal.h"

#include <math.h>

namespace ea {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kNegInf = -__builtin_huge_valf();

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint16_t bf16_t;  // bfloat16 storage

__device__ __forceinline__ float bf_bits_to_f(uint32_t bits16) { return __uint_as_float(bits16 << 16); }
// Two floats to packed bfloat16 (round to nearest even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

template <typename T>
struct Num;
template <>
struct Num<float> {
  static __device__ __forceinline__ float ld(const float* p) { return *p; }
  static __device__ __forceinline__ float rnd(float v) { return v; }
  static __device__ __forceinline__ void st(float* p, float v) { *p = v; }
};
template <>
struct Num<bf16_t> {
  static __device__ __forceinline__ float ld(const bf16_t* p) { return bf_bits_to_f(*p); }
  static __device__ __forceinline__ float rnd(float v) { return bf_bits_to_f(pack_bf2(v, 0.f) & 0xffffu); }
  static __device__ __forceinline__ void st(bf16_t* p, float v) { *p = (bf16_t)(pack_bf2(v, 0.f) & 0xffffu); }
};

template <typename T>
__device__ __forceinline__ float ld_or0(const void* p, size_t k) {
  return p ? Num<T>::ld(static_cast<const T*>(p) + k) : 0.f;
}

// Q consecutive elements of type T held by one lane, packed in dwords.
template <typename T, int Q>
struct Frag {
  static constexpr int ND = Q * (int)sizeof(T) / 4;
  static_assert(ND == 1 || ND == 2 || ND % 4 == 0, "fragment size");
  uint32_t w[ND];

  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int k = 0; k < ND; ++k) w[k] = 0u;
  }
  __device__ __forceinline__ void load(const T* p) {
    if constexpr (ND % 4 == 0) {
      const u32x4* q = reinterpret_cast<const u32x4*>(p);
#pragma unroll
      for (int s = 0; s < ND / 4; ++s) {
        const u32x4 v = q[s];
        w[4 * s] = v.x; w[4 * s + 1] = v.y; w[4 * s + 2] = v.z; w[4 * s + 3] = v.w;
      }
    } else if constexpr (ND == 2) {
      const u32x2 v = *reinterpret_cast<const u32x2*>(p);
      w[0] = v.x; w[1] = v.y;
    } else {
      w[0] = *reinterpret_cast<const uint32_t*>(p);
    }
  }
  __device__ __forceinline__ void store(T* p) const {
    if constexpr (ND % 4 == 0) {
      u32x4* q = reinterpret_cast<u32x4*>(p);
#pragma unroll
      for (int s = 0; s < ND / 4; ++s) q[s] = u32x4{w[4 * s], w[4 * s + 1], w[4 * s + 2], w[4 * s + 3]};
    } else if constexpr (ND == 2) {
      *reinterpret_cast<u32x2*>(p) = u32x2{w[0], w[1]};
    } else {
      *reinterpret_cast<uint32_t*>(p) = w[0];
    }
  }
  __device__ __forceinline__ float get(int k) const {
    if constexpr (sizeof(T) == 4) {
      return __uint_as_float(w[k]);
    } else {
      return (k & 1) ? __uint_as_float(w[k >> 1] & 0xffff0000u) : __uint_as_float(w[k >> 1] << 16);
    }
  }
  // From Q floats; bfloat16 fragments round to nearest even.
  __device__ __forceinline__ void set(const float* v) {
    if constexpr (sizeof(T) == 4) {
#pragma unroll
      for (int k = 0; k < Q; ++k) w[k] = __float_as_uint(v[k]);
    } else {
#pragma unroll
      for (int k = 0; k < ND; ++k) w[k] = pack_bf2(v[2 * k], v[2 * k + 1]);
    }
  }
};

// acc += A * B over one fragment pair (see the operand convention above).
template <int Q>
__device__ __forceinline__ f32x4 mma(f32x4 acc, const Frag<bf16_t, Q>& a, const Frag<bf16_t, Q>& b) {
  if constexpr (Q % 8 == 0) {
#pragma unroll
    for (int s = 0; s < Q / 8; ++s) {
      const u32x4 av = {a.w[4 * s], a.w[4 * s + 1], a.w[4 * s + 2], a.w[4 * s + 3]};
      const u32x4 bv = {b.w[4 * s], b.w[4 * s + 1], b.w[4 * s + 2], b.w[4 * s + 3]};
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av),
                                                    __builtin_bit_cast(bf16x8, bv), acc, 0, 0, 0);
    }
  } else {
    static_assert(Q == 4, "bfloat16 fragments hold 4 or a multiple of 8 values");
    const u32x2 av = {a.w[0], a.w[1]};
    const u32x2 bv = {b.w[0], b.w[1]};
    acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, av),
                                                   __builtin_bit_cast(i16x4, bv), acc, 0, 0, 0);
  }
  return acc;
}
template <int Q>
__device__ __forceinline__ f32x4 mma(f32x4 acc, const Frag<float, Q>& a, const Frag<float, Q>& b) {
#pragma unroll
  for (int s = 0; s < Q; ++s)
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w[s]), __uint_as_float(b.w[s]), acc, 0, 0, 0);
  return acc;
}

__device__ __forceinline__ float wave_max_lg(float v) {  // max over the 4 lane groups of a column
  v = fmaxf(v, __shfl_xor(v, 16));
  return fmaxf(v, __shfl_xor(v, 32));
}
__device__ __forceinline__ float wave_sum_lg(float v) {
  v += __shfl_xor(v, 16);
  return v + __shfl_xor(v, 32);
}

// ------------------------------------------------------------------ QKV

// Q | K | V = X W^T + b for rows (b, i) of the padded batch; rows of padded
// nodes and the slots i in [n, NP) are written as zeros. Q, K: [B, H, NP, DH];
// V transposed: [B, H, DH, NP]. Grid: (ceil(B*NP/64), 3*D/64), 4 waves of 16 rows.
template <typename T, int D, int DH>
__global__ __launch_bounds__(kThreads) void qkv_kernel(LayerArgs a) {
  constexpr int H = D / DH;
  constexpr int Qk = D / 4;                    // contraction quarter per lane group
  constexpr int CQ = sizeof(T) == 2 ? 8 : 4;   // elements per 16-byte step
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, li = l & 15, lg = l >> 4;
  const int NP = a.NP, n = a.n;
  const long rows = (long)a.B * NP;
  const long m0 = (long)blockIdx.x * 64 + w * 16;
  const int f0 = blockIdx.y * 64;
  const int which = f0 / D, fl0 = f0 % D;
  const T* W = static_cast<const T*>(which == 0 ? a.w_q : which == 1 ? a.w_k : a.w_v);
  const void* bias = which == 0 ? a.b_q : which == 1 ? a.b_k : a.b_v;

  const long m = m0 + li;
  bool valid = false;
  const T* xrow = static_cast<const T*>(a.X);
  if (m < rows) {
    const int b = (int)(m / NP), i = (int)(m % NP);
    if (i < n && a.mask[(size_t)b * n + i]) {
      valid = true;
      xrow += ((size_t)b * n + i) * D;
    }
  }
  f32x4 acc[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < Qk / CQ; ++s) {
    Frag<T, CQ> xa;
    if (valid) xa.load(xrow + lg * Qk + s * CQ); else xa.zero();
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      Frag<T, CQ> wb;
      wb.load(W + (size_t)(fl0 + nt * 16 + li) * D + lg * Qk + s * CQ);
      acc[nt] = mma(acc[nt], xa, wb);
    }
  }
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int fl = fl0 + nt * 16 + li, h = fl / DH, t = fl % DH;
    const float bv = ld_or0<T>(bias, fl);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const long mr = m0 + 4 * lg + r;
      if (mr >= rows) continue;
      const int b = (int)(mr / NP), i = (int)(mr % NP);
      const bool ok = i < n && a.mask[(size_t)b * n + i];
      const float v = ok ? acc[nt][r] + bv : 0.f;
      if (which == 2)
        Num<T>::st(static_cast<T*>(a.Vt) + (((size_t)b * H + h) * DH + t) * NP + i, v);
      else
        Num<T>::st(static_cast<T*>(which == 0 ? a.Qw : a.Kw) + (((size_t)b * H + h) * NP + i) * DH + t, v);
    }
  }
}

// ------------------------------------------------------------------ score stage

// Per-lane state of one (graph b, 16-query block) for the score stage.
template <typename T, int H, int DH, int DE>
struct Scorer {
  int b, n, NP, JT, i, li, lg;
  bool mi;
  const uint8_t* mask_b;
  const T* E;
  const T* Kw;
  float scale;
  Frag<T, DH / 4> qf[H];
  Frag<T, DE / 4> wf;  // edge-FiLM weights, row li: gamma of head li, then beta of head li-H
  float bmul[H], badd[H];
  float gy[2 * H];     // gamma_y (1 + ...) then beta_y, for graph b

  // Must be called by every thread of the block (contains a barrier).
  __device__ __forceinline__ void init(const LayerArgs& a, int b_, int i0, float* gy_s) {
    const int tid = threadIdx.x, l = tid & 63;
    li = l & 15; lg = l >> 4;
    b = b_; n = a.n; NP = a.NP; JT = a.NP / 16; i = i0 + li;
    mask_b = a.mask + (size_t)b * n;
    mi = i < n && mask_b[i];
    E = static_cast<const T*>(a.E);
    Kw = static_cast<const T*>(a.Kw);
    scale = a.scale;
    // global FiLM of graph b: one thread per coefficient
    if (tid < 2 * H) {
      const int o = tid, h = o % H;
      const bool mul = o < H;
      const T* Wy = static_cast<const T*>(mul ? a.w_ymul : a.w_yadd) + (size_t)h * a.dy;
      const T* yb = static_cast<const T*>(a.y) + (size_t)b * a.dy;
      float acc = ld_or0<T>(mul ? a.b_ymul : a.b_yadd, h);
      for (int c = 0; c < a.dy; ++c) acc += Num<T>::ld(yb + c) * Num<T>::ld(Wy + c);
      gy_s[o] = mul ? 1.f + acc : acc;
    }
    const T* Qw = static_cast<const T*>(a.Qw);
#pragma unroll
    for (int h = 0; h < H; ++h) qf[h].load(Qw + (((size_t)b * H + h) * NP + i) * DH + lg * (DH / 4));
    if (li < H)
      wf.load(static_cast<const T*>(a.w_emul) + (size_t)li * DE + lg * (DE / 4));
    else if (li < 2 * H)
      wf.load(static_cast<const T*>(a.w_eadd) + (size_t)(li - H) * DE + lg * (DE / 4));
    else
      wf.zero();
#pragma unroll
    for (int h = 0; h < H; ++h) {
      bmul[h] = ld_or0<T>(a.b_emul, h);
      badd[h] = ld_or0<T>(a.b_eadd, h);
    }
    __syncthreads();
#pragma unroll
    for (int o = 0; o < 2 * H; ++o) gy[o] = gy_s[o];
  }

  // Masked logits u[h][r] of query i for key j = 16*jt + 4*lg + r. Every
  // thread of the block must call this the same number of times (barriers);
  // a tile jt >= JT yields -inf. fs: this wave's 16*16*16-float scratch.
  __device__ __forceinline__ void logits(int jt, float (&u)[H][4], float* fs) const {
    const int j0 = 16 * jt;
    const bool tile = jt < JT;
    // edge FiLM for the 16 keys of the tile; MFMA column = query row
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) {
      const int j = j0 + jj;
      Frag<T, DE / 4> ef;
      if (mi && j < n && mask_b[j])
        ef.load(E + (((size_t)b * n + i) * n + j) * DE + lg * (DE / 4));
      else
        ef.zero();
      const f32x4 F = mma(f32x4{0.f, 0.f, 0.f, 0.f}, wf, ef);
      *reinterpret_cast<f32x4*>(fs + (jj * 16 + li) * 16 + 4 * lg) = F;
    }
    __syncthreads();
    float gam[H][4], bet[H][4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float* src = fs + ((4 * lg + r) * 16 + li) * 16;
#pragma unroll
      for (int h = 0; h < H; ++h) {
        gam[h][r] = 1.f + (src[h] + bmul[h]);
        bet[h][r] = src[H + h] + badd[h];
      }
    }
    __syncthreads();
    bool real[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = j0 + 4 * lg + r;
      real[r] = mi && j < n && mask_b[j];
    }
#pragma unroll
    for (int h = 0; h < H; ++h) {
      Frag<T, DH / 4> kf;
      if (tile) kf.load(Kw + (((size_t)b * H + h) * NP + j0 + li) * DH + lg * (DH / 4));
      else kf.zero();
      const f32x4 s = mma(f32x4{0.f, 0.f, 0.f, 0.f}, kf, qf[h]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float v = ((s[r] * scale) * gam[h][r] + bet[h][r]) * gy[h] + gy[H + h];
        u[h][r] = real[r] ? v : kNegInf;
      }
    }
  }
};

// ------------------------------------------------------------------ edge update

// Residual edge update of one 16x16 (query, key) tile from the attention map
// staged in LDS as [key jj][query li][head]. MFMA per key j and 16-channel
// chunk: E'^T (channels x queries) = W_e (channels x heads) A^T + E^T + b_e.
template <typename T, int H, int DE>
struct Updater {
  static constexpr int QH = sizeof(T) == 2 ? 4 : H / 4;  // heads per lane group
  static constexpr int NCH = DE / 16;
  Frag<T, QH> wef[NCH];
  float be[DE / 4];
  bool has_heads;

  __device__ __forceinline__ void init(const LayerArgs& a, int li, int lg) {
    const T* We = static_cast<const T*>(a.w_e);
    has_heads = lg * QH < H;
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
      // MFMA row li of chunk ch is channel (li/4)*(DE/4) + 4*ch + li%4, so that
      // output rows 4*lg + r land on this lane group's channel quarter.
      const int c = (li >> 2) * (DE / 4) + 4 * ch + (li & 3);
      if (has_heads) wef[ch].load(We + (size_t)c * H + lg * QH); else wef[ch].zero();
    }
#pragma unroll
    for (int k = 0; k < DE / 4; ++k) be[k] = ld_or0<T>(a.b_e, lg * (DE / 4) + k);
  }

  __device__ __forceinline__ void tile(const T* E, T* Eout, int b, int n, int i, bool mi,
                                       const uint8_t* mask_b, int j0, int li, int lg,
                                       const T* stage) const {
#pragma unroll 4
    for (int jj = 0; jj < 16; ++jj) {
      const int j = j0 + jj;
      const bool inb = i < n && j < n;
      const bool real = mi && j < n && mask_b[j];
      Frag<T, QH> af;
      if (has_heads) af.load(stage + (jj * 16 + li) * H + lg * QH); else af.zero();
      const size_t off = (((size_t)b * n + i) * n + j) * DE + lg * (DE / 4);
      Frag<T, DE / 4> ef;
      if (real) ef.load(E + off); else ef.zero();
      float out[DE / 4];
#pragma unroll
      for (int ch = 0; ch < NCH; ++ch) {
        f32x4 c = {ef.get(4 * ch) + be[4 * ch], ef.get(4 * ch + 1) + be[4 * ch + 1],
                   ef.get(4 * ch + 2) + be[4 * ch + 2], ef.get(4 * ch + 3) + be[4 * ch + 3]};
        c = mma(c, wef[ch], af);
#pragma unroll
        for (int r = 0; r < 4; ++r) out[4 * ch + r] = real ? c[r] : 0.f;
      }
      if (inb) {
        Frag<T, DE / 4> of;
        of.set(out);
        of.store(Eout + off);
      }
    }
  }
};

// Stage this lane's A values (keys 4*lg + r, all heads) as [key][query][head].
template <typename T, int H>
__device__ __forceinline__ void stage_A(T* sw, const float (&A)[H][4], int li, int lg) {
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float hv[H];
#pragma unroll
    for (int h = 0; h < H; ++h) hv[h] = A[h][r];
    Frag<T, H> f;
    f.set(hv);
    f.store(sw + ((4 * lg + r) * 16 + li) * H);
  }
}

// Cross-wave reduction of the per-wave O^T partials and the store of O rows.
template <typename T, int H, int DH>
__device__ __forceinline__ void reduce_store_O(const LayerArgs& a, float* os, const f32x4 (&oacc)[H][DH / 16],
                                               int b, int i0, int w, int li, int lg) {
  constexpr int D = H * DH;
  __syncthreads();
#pragma unroll
  for (int h = 0; h < H; ++h)
#pragma unroll
    for (int tc = 0; tc < DH / 16; ++tc)
#pragma unroll
      for (int r = 0; r < 4; ++r) os[((w * D) + h * DH + tc * 16 + 4 * lg + r) * 16 + li] = oacc[h][tc][r];
  __syncthreads();
  const uint8_t* mask_b = a.mask + (size_t)b * a.n;
  for (int idx = threadIdx.x; idx < 16 * D; idx += kThreads) {
    const int il = idx / D, c = idx % D, ii = i0 + il;
    if (ii >= a.n) continue;
    float v = 0.f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) v += os[(ww * D + c) * 16 + il];
    if (!mask_b[ii]) v = 0.f;
    Num<T>::st(static_cast<T*>(a.O) + ((size_t)b * a.n + ii) * D + c, v);
  }
}

// ------------------------------------------------------------------ attention

// One block per (graph b = blockIdx.y, 16-query block blockIdx.x); wave w
// owns key tiles w, w+4, ... . kSingle/kFused/kLogits keep the MAXT logit
// tiles of a wave in registers (n <= 64*MAXT); kOnline streams any n.
template <typename T, int H, int DH, int DE, int MAXT, int MODE>
__global__ __launch_bounds__(kThreads) void attn_kernel(LayerArgs a) {
  constexpr int D = H * DH;
  static_assert(D <= 256 && 2 * H <= 16, "shape");
  __shared__ __align__(16) float scratch[kWaves * 16 * 16 * 16];  // FiLM transpose, then O reduction
  __shared__ float red_s[2][kWaves][H][16];
  __shared__ float gy_s[2 * H];
  __shared__ __align__(16) T stage_s[MODE == kFused ? kWaves * 16 * 16 * H : 8];

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, li = l & 15, lg = l >> 4;
  const int b = blockIdx.y, i0 = blockIdx.x * 16;
  Scorer<T, H, DH, DE> sc;
  sc.init(a, b, i0, gy_s);
  float* fs = scratch + w * 4096;
  const int JT = sc.JT, n = a.n, NP = a.NP, i = sc.i;
  const T* Vt = static_cast<const T*>(a.Vt);

  f32x4 oacc[H][DH / 16];
#pragma unroll
  for (int h = 0; h < H; ++h)
#pragma unroll
    for (int tc = 0; tc < DH / 16; ++tc) oacc[h][tc] = f32x4{0.f, 0.f, 0.f, 0.f};

  if constexpr (MODE == kOnline) {
    float m_run[H], l_run[H];
#pragma unroll
    for (int h = 0; h < H; ++h) { m_run[h] = kNegInf; l_run[h] = 0.f; }
    const int NT = (JT + kWaves - 1) / kWaves;
    for (int tt = 0; tt < NT; ++tt) {
      const int jt = w + kWaves * tt;
      float u[H][4];
      sc.logits(jt, u, fs);
      if (jt < JT) {
        const int j0 = 16 * jt;
#pragma unroll
        for (int h = 0; h < H; ++h) {
          const float tm = wave_max_lg(fmaxf(fmaxf(u[h][0], u[h][1]), fmaxf(u[h][2], u[h][3])));
          const float mnew = fmaxf(m_run[h], tm);
          const float alpha = (mnew == kNegInf) ? 1.f : __expf(m_run[h] - mnew);
          float p[4], ps = 0.f;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            p[r] = (u[h][r] == kNegInf) ? 0.f : __expf(u[h][r] - mnew);
            ps += p[r];
          }
          l_run[h] = l_run[h] * alpha + ps;
          m_run[h] = mnew;
          Frag<T, 4> af;
          af.set(p);
#pragma unroll
          for (int tc = 0; tc < DH / 16; ++tc) {
            Frag<T, 4> vf;
            vf.load(Vt + (((size_t)b * H + h) * DH + tc * 16 + li) * NP + j0 + 4 * lg);
            oacc[h][tc] *= alpha;
            oacc[h][tc] = mma(oacc[h][tc], vf, af);
          }
        }
      }
    }
    // combine lane groups, then waves
#pragma unroll
    for (int h = 0; h < H; ++h) {
      const float lsum = wave_sum_lg(l_run[h]);
      if (lg == 0) { red_s[0][w][h][li] = m_run[h]; red_s[1][w][h][li] = lsum; }
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < H; ++h) {
      float M = kNegInf;
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, red_s[0][ww][h][li]);
      float L = 0.f;
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) {
        const float mw = red_s[0][ww][h][li];
        L += (mw == kNegInf) ? 0.f : red_s[1][ww][h][li] * __expf(mw - M);
      }
      const float f = (m_run[h] == kNegInf || !(L > 0.f)) ? 0.f : __expf(m_run[h] - M) / L;
#pragma unroll
      for (int tc = 0; tc < DH / 16; ++tc) oacc[h][tc] *= f;
      if (w == 0 && lg == 0) a.lse[((size_t)b * H + h) * NP + i] = (L > 0.f) ? M + __logf(L) : kNegInf;
    }
    reduce_store_O<T, H, DH>(a, scratch, oacc, b, i0, w, li, lg);
  } else {
    float u[MAXT][H][4];
#pragma unroll
    for (int tt = 0; tt < MAXT; ++tt) sc.logits(w + kWaves * tt, u[tt], fs);

    if constexpr (MODE == kLogits) {
      if (i < n) {
#pragma unroll
        for (int tt = 0; tt < MAXT; ++tt)
#pragma unroll
          for (int h = 0; h < H; ++h)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int j = 16 * (w + kWaves * tt) + 4 * lg + r;
              if (j < n) a.U[(((size_t)b * H + h) * n + i) * n + j] = u[tt][h][r];
            }
      }
      return;
    } else {
      // masked softmax over the full row: max, then sum, across lane groups and waves
#pragma unroll
      for (int h = 0; h < H; ++h) {
        float m = kNegInf;
#pragma unroll
        for (int tt = 0; tt < MAXT; ++tt)
#pragma unroll
          for (int r = 0; r < 4; ++r) m = fmaxf(m, u[tt][h][r]);
        m = wave_max_lg(m);
        if (lg == 0) red_s[0][w][h][li] = m;
      }
      __syncthreads();
      float inv[H];
#pragma unroll
      for (int h = 0; h < H; ++h) {
        float M = kNegInf;
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, red_s[0][ww][h][li]);
        float s = 0.f;
#pragma unroll
        for (int tt = 0; tt < MAXT; ++tt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float p = (u[tt][h][r] == kNegInf) ? 0.f : __expf(u[tt][h][r] - M);
            u[tt][h][r] = p;
            s += p;
          }
        s = wave_sum_lg(s);
        if (lg == 0) red_s[1][w][h][li] = s;
      }
      __syncthreads();
#pragma unroll
      for (int h = 0; h < H; ++h) {
        float L = 0.f;
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) L += red_s[1][ww][h][li];
        inv[h] = (L > 0.f) ? 1.f / L : 0.f;
      }
      // A (rounded to the storage type), its store, and O^T += V^T A^T
      T* Ag = static_cast<T*>(a.A);
#pragma unroll
      for (int tt = 0; tt < MAXT; ++tt) {
        const int jt = w + kWaves * tt, j0 = 16 * jt;
#pragma unroll
        for (int h = 0; h < H; ++h)
#pragma unroll
          for (int r = 0; r < 4; ++r) u[tt][h][r] = Num<T>::rnd(u[tt][h][r] * inv[h]);
        if (jt < JT) {
          if (i < n) {
#pragma unroll
            for (int h = 0; h < H; ++h) {
              T* row = Ag + (((size_t)b * H + h) * n + i) * n;
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const int j = j0 + 4 * lg + r;
                if (j < n) Num<T>::st(row + j, u[tt][h][r]);
              }
            }
          }
#pragma unroll
          for (int h = 0; h < H; ++h) {
            Frag<T, 4> af;
            af.set(u[tt][h]);
#pragma unroll
            for (int tc = 0; tc < DH / 16; ++tc) {
              Frag<T, 4> vf;
              vf.load(Vt + (((size_t)b * H + h) * DH + tc * 16 + li) * NP + j0 + 4 * lg);
              oacc[h][tc] = mma(oacc[h][tc], vf, af);
            }
          }
        }
      }
      if constexpr (MODE == kFused) {
        Updater<T, H, DE> up;
        up.init(a, li, lg);
        T* sw = stage_s + w * 16 * 16 * H;
#pragma unroll
        for (int tt = 0; tt < MAXT; ++tt) {
          const int jt = w + kWaves * tt;
          stage_A<T, H>(sw, u[tt], li, lg);
          __syncthreads();
          if (jt < JT)
            up.tile(sc.E, static_cast<T*>(a.E_out), b, n, i, sc.mi, sc.mask_b, 16 * jt, li, lg, sw);
          __syncthreads();
        }
      }
      reduce_store_O<T, H, DH>(a, scratch, oacc, b, i0, w, li, lg);
    }
  }
}

// ------------------------------------------------------------------ update kernel

// Grid (NP/16 query blocks, B, ceil(NP/64)); wave w of block z takes key tile
// 4*z + w. kReadA reads A from the forward's output; kRecompute re-runs the
// score stage and takes A = exp(u - lse) from pass 1's statistics.
template <typename T, int H, int DH, int DE, int MODE>
__global__ __launch_bounds__(kThreads) void update_kernel(LayerArgs a) {
  __shared__ __align__(16) float scratch[MODE == kRecompute ? kWaves * 16 * 16 * 16 : 4];
  __shared__ float gy_s[2 * H];
  __shared__ __align__(16) T stage_s[kWaves * 16 * 16 * H];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, li = l & 15, lg = l >> 4;
  const int b = blockIdx.y, i0 = blockIdx.x * 16, i = i0 + li;
  const int n = a.n, NP = a.NP, JT = NP / 16;
  const int jt = blockIdx.z * kWaves + w, j0 = 16 * jt;
  const uint8_t* mask_b = a.mask + (size_t)b * n;
  const bool mi = i < n && mask_b[i];
  float A[H][4];
  if constexpr (MODE == kRecompute) {
    Scorer<T, H, DH, DE> sc;
    sc.init(a, b, i0, gy_s);
    float u[H][4];
    sc.logits(jt, u, scratch + w * 4096);
#pragma unroll
    for (int h = 0; h < H; ++h) {
      const float L = a.lse[((size_t)b * H + h) * NP + i];
#pragma unroll
      for (int r = 0; r < 4; ++r)
        A[h][r] = (u[h][r] == kNegInf || L == kNegInf) ? 0.f : Num<T>::rnd(__expf(u[h][r] - L));
    }
  } else {
    const T* Ag = static_cast<const T*>(a.A);
#pragma unroll
    for (int h = 0; h < H; ++h)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = j0 + 4 * lg + r;
        A[h][r] = (jt < JT && i < n && j < n) ? Num<T>::ld(Ag + (((size_t)b * H + h) * n + i) * n + j) : 0.f;
      }
  }
  Updater<T, H, DE> up;
  up.init(a, li, lg);
  T* sw = stage_s + w * 16 * 16 * H;
  stage_A<T, H>(sw, A, li, lg);
  __syncthreads();
  if (jt < JT)
    up.tile(static_cast<const T*>(a.E), static_cast<T*>(a.E_out), b, n, i, mi, mask_b, j0, li, lg, sw);
}

// ------------------------------------------------------------------ dispatch

template <typename T, int H, int DH, int DE, int MODE>
hipError_t attn_maxt(const LayerArgs& a, int maxt, dim3 grid, hipStream_t s) {
  switch (maxt) {
    case 1: hipLaunchKernelGGL((attn_kernel<T, H, DH, DE, 1, MODE>), grid, dim3(kThreads), 0, s, a); break;
    case 2: hipLaunchKernelGGL((attn_kernel<T, H, DH, DE, 2, MODE>), grid, dim3(kThreads), 0, s, a); break;
    case 3: hipLaunchKernelGGL((attn_kernel<T, H, DH, DE, 3, MODE>), grid, dim3(kThreads), 0, s, a); break;
    case 4: hipLaunchKernelGGL((attn_kernel<T, H, DH, DE, 4, MODE>), grid, dim3(kThreads), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T, int H, int DH, int DE>
hipError_t attn_shape(const LayerArgs& a, int mode, hipStream_t s) {
  const int JT = a.NP / 16;
  const dim3 grid(JT, a.B);
  const int maxt = (JT + kWaves - 1) / kWaves;
  switch (mode) {
    case kSingle: return attn_maxt<T, H, DH, DE, kSingle>(a, maxt, grid, s);
    case kFused: return attn_maxt<T, H, DH, DE, kFused>(a, maxt, grid, s);
    case kLogits: return attn_maxt<T, H, DH, DE, kLogits>(a, maxt, grid, s);
    case kOnline:
      hipLaunchKernelGGL((attn_kernel<T, H, DH, DE, 1, kOnline>), grid, dim3(kThreads), 0, s, a);
      return hipGetLastError();
    default: return hipErrorInvalidValue;
  }
}

template <typename T, int H, int DH, int DE>
hipError_t update_shape(const LayerArgs& a, int mode, hipStream_t s) {
  const int JT = a.NP / 16;
  const dim3 grid(JT, a.B, (JT + kWaves - 1) / kWaves);
  if (mode == kReadA)
    hipLaunchKernelGGL((update_kernel<T, H, DH, DE, kReadA>), grid, dim3(kThreads), 0, s, a);
  else if (mode == kRecompute)
    hipLaunchKernelGGL((update_kernel<T, H, DH, DE, kRecompute>), grid, dim3(kThreads), 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

template <typename T, int D, int DH>
hipError_t qkv_shape(const LayerArgs& a, hipStream_t s) {
  const long rows = (long)a.B * a.NP;
  const dim3 grid((unsigned)((rows + 63) / 64), 3 * D / 64);
  hipLaunchKernelGGL((qkv_kernel<T, D, DH>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

bool shape_supported(int dtype, int H, int dh, int de) {
  if (dtype != 0 && dtype != 1) return false;
  return (H == 4 && dh == 16 && de == 16) || (H == 8 && dh == 32 && de == 64);
}

#define EA_SHAPES(CALL, T)                                          \
  if (H == 4 && dh == 16 && de == 16) return CALL(T, 4, 16, 16);    \
  if (H == 8 && dh == 32 && de == 64) return CALL(T, 8, 32, 64);

hipError_t launch_qkv(const LayerArgs& a, int dtype, int H, int dh, int de, hipStream_t s) {
#define EA_QKV(T, HH, DHH, DEE) qkv_shape<T, HH * DHH, DHH>(a, s)
  if (dtype == 0) { EA_SHAPES(EA_QKV, float) }
  else { EA_SHAPES(EA_QKV, bf16_t) }
#undef EA_QKV
  return hipErrorInvalidValue;
}

hipError_t launch_attn(const LayerArgs& a, int dtype, int H, int dh, int de, int mode, hipStream_t s) {
#define EA_ATT(T, HH, DHH, DEE) attn_shape<T, HH, DHH, DEE>(a, mode, s)
  if (dtype == 0) { EA_SHAPES(EA_ATT, float) }
  else { EA_SHAPES(EA_ATT, bf16_t) }
#undef EA_ATT
  return hipErrorInvalidValue;
}

hipError_t launch_update(const LayerArgs& a, int dtype, int H, int dh, int de, int mode, hipStream_t s) {
#define EA_UPD(T, HH, DHH, DEE) update_shape<T, HH, DHH, DEE>(a, mode, s)
  if (dtype == 0) { EA_SHAPES(EA_UPD, float) }
  else { EA_SHAPES(EA_UPD, bf16_t) }
#undef EA_UPD
  return hipErrorInvalidValue;
}

}  // namespace ea
