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
#include "ea_device.h"

#include <math.h>

namespace ea {
namespace {

// Bit jj set when key j0 + jj is a real node, from the mask byte this lane
// loaded for key j0 + li (identical in all lanes).
__device__ __forceinline__ uint32_t key_bits(uint32_t mask_byte) {
  return (uint32_t)(__ballot(mask_byte != 0u) & 0xffffull);
}

// Logical (16-query block, graph) of this block. Consecutive block ids go to
// the 8 XCDs in turn; regrouping them keeps all query blocks of a graph on one
// XCD, whose L2 then serves the graph's K and V to all of them.
__device__ __forceinline__ void xcd_block(int& ib, int& b) {
  const int IB = gridDim.x, NB = gridDim.x * gridDim.y;
  const int L = blockIdx.y * gridDim.x + blockIdx.x;
  if ((NB & 7) == 0) {
    const int u = (L & 7) * (NB >> 3) + (L >> 3);
    ib = u % IB;
    b = u / IB;
  } else {
    ib = blockIdx.x;
    b = blockIdx.y;
  }
}

// Lane-group block transpose in registers. Lane group p (lanes 16p..16p+15)
// holds in R[x] the block (p, x); afterwards it holds in R[x] the block
// (x, p). Two rounds of swaps: v_permlane32_swap exchanges lane groups
// {0,1} <-> {2,3} (bit 1 of the group), v_permlane16_swap exchanges 0 <-> 1
// and 2 <-> 3 (bit 0). NE is the number of 32-bit elements per block.
template <int NE>
__device__ __forceinline__ void lane_group_transpose(float (&R)[4][NE]) {
#pragma unroll
  for (int e = 0; e < NE; ++e) {
    float s[2][2];  // s[x0][bit1 of the source block's second coordinate]
#pragma unroll
    for (int x0 = 0; x0 < 2; ++x0) {
      const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(R[x0][e]), __float_as_uint(R[x0 ^ 2][e]),
                                                      false, false);
      s[x0][0] = __uint_as_float(p[0]);
      s[x0][1] = __uint_as_float(p[1]);
    }
#pragma unroll
    for (int b1 = 0; b1 < 2; ++b1) {
      const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(s[0][b1]), __float_as_uint(s[1][b1]),
                                                      false, false);
      R[2 * b1][e] = __uint_as_float(p[0]);
      R[2 * b1 + 1][e] = __uint_as_float(p[1]);
    }
  }
}

// ------------------------------------------------------------------ QKV

// Global FiLM coefficients gamma_y = 1 + W_ymul y + b_ymul and
// beta_y = W_yadd y + b_yadd of the graphs whose slot 0 lies in rows
// [m0, m0 + mrows) of the padded batch; 16 lanes per coefficient (2H <= 16),
// loads batched.
// Without score modulation they are 1 and 0 and y is not read.
template <typename T, int H>
__device__ __forceinline__ void global_film(const LayerArgs& a, uint32_t m0, uint32_t mrows, uint32_t rows) {
  const uint32_t NP = a.NP;
  const int tid = threadIdx.x, o = tid >> 4, part = tid & 15;
  if (a.variant & kNoScoreMod) {
    for (uint32_t m = (m0 + NP - 1) / NP * NP; m < m0 + mrows && m < rows; m += NP)
      if (o < 2 * H && part == 0) a.gy[(size_t)(m / NP) * 2 * H + o] = o < H ? 1.f : 0.f;
    return;
  }
  const T* Wy = static_cast<const T*>(o < H ? a.w_ymul : a.w_yadd) + (size_t)(o % H) * a.dy;
  for (uint32_t m = (m0 + NP - 1) / NP * NP; m < m0 + mrows && m < rows; m += NP) {
    const uint32_t b = m / NP;
    const T* yb = static_cast<const T*>(a.y) + (size_t)b * a.dy;
    float acc = 0.f;
    if (o < 2 * H) {
      constexpr int kBatch = 8;
      for (int c0 = 0; c0 < a.dy; c0 += 16 * kBatch) {
        float yv[kBatch], wv[kBatch];
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
          const int c = c0 + part + 16 * k;
          const float yl = Num<T>::ld(yb + (c < a.dy ? c : 0));
          const float wl = Num<T>::ld(Wy + (c < a.dy ? c : 0));
          yv[k] = c < a.dy ? yl : 0.f;
          wv[k] = c < a.dy ? wl : 0.f;
        }
#pragma unroll
        for (int k = 0; k < kBatch; ++k) acc += yv[k] * wv[k];
      }
    }
    acc += __shfl_xor(acc, 1);
    acc += __shfl_xor(acc, 2);
    acc += __shfl_xor(acc, 4);
    acc += __shfl_xor(acc, 8);
    if (o < 2 * H && part == 0) {
      const float bias = ld_or0<T>(o < H ? a.b_ymul : a.b_yadd, o % H);
      a.gy[(size_t)b * 2 * H + o] = o < H ? 1.f + (bias + acc) : bias + acc;
    }
  }
}

// Most logical blocks the work order sorts (one byte of LDS each); larger
// batches keep the plain order.
constexpr int kOrderMax = 16384;
constexpr int kOrderKeys = 6;  // 0, and 1 + 0..4 live tiles per wave

// Work order of fused_stream_kernel (a.order): its logical blocks (graph,
// 16-query block) sorted by expected length, longest first, equal lengths in
// index order.
// The hardware deals block ids to the 8 XCDs in turn and each XCD starts its
// blocks in id order, so every XCD gets the same mix of long and short
// blocks and starts the longest ones first (with a prefix node mask the
// blocks of a ragged batch range from one key tile to several per wave). A
// block's length is taken as 1 + the most key tiles with a real key that one
// of its waves reads (wave w reads tiles w, w + kWaves, ...), and 0 without a
// real query. One block of threads; smem: kOrderMax + 128 bytes.
__device__ __forceinline__ void work_order(const LayerArgs& a, unsigned char* smem) {
  const int n = a.n, JT = a.NP / 16, NB = a.B * JT;
  uint8_t* real_s = smem;  // per (graph, 16-node group): some real node
  int* cnt_s = reinterpret_cast<int*>(smem + kOrderMax);
  int* wcnt_s = cnt_s + kOrderKeys;  // [kWaves][kOrderKeys]
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  // a 16-node group is a query block and a key tile at once
  for (int p = tid; p < NB; p += kThreads) {
    const int b = p / JT, t = p % JT;
    uint32_t m[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int j = 16 * t + r;
      m[r] = a.mask[(size_t)b * n + (j < n ? j : n - 1)];
    }
    uint32_t any = 0u;
#pragma unroll
    for (int r = 0; r < 16; ++r) any |= (16 * t + r < n) ? m[r] : 0u;
    real_s[p] = any != 0u;
  }
  if (tid < kOrderKeys) cnt_s[tid] = 0;
  __syncthreads();
  auto key_of = [&](int L) -> int {
    if (!real_s[L]) return 0;
    const uint8_t* g = real_s + (L / JT) * JT;
    int most = 0;
    for (int ww = 0; ww < kWaves; ++ww) {
      int c = 0;
      for (int jt = ww; jt < JT; jt += kWaves) c += g[jt];
      most = c > most ? c : most;
    }
    return 1 + (most < kOrderKeys - 2 ? most : kOrderKeys - 2);
  };
  for (int L = tid; L < NB; L += kThreads) atomicAdd(&cnt_s[key_of(L)], 1);
  __syncthreads();
  // next position of each key: longer blocks first (the blocks without a
  // real query, zero stores only, last: placed right after the longest ones
  // instead, they shared the first round's bandwidth with them and the
  // kernel took as long)
  int start[kOrderKeys];
  {
    int acc = 0;
#pragma unroll
    for (int k = kOrderKeys - 1; k >= 0; --k) {
      start[k] = acc;
      acc += cnt_s[k];
    }
  }
  const uint64_t below = (l == 0) ? 0ull : (~0ull >> (64 - l));  // lanes under this one
  for (int c0 = 0; c0 < NB; c0 += kThreads) {
    const int L = c0 + tid;
    const int k = L < NB ? key_of(L) : -1;
    int rank = 0;
#pragma unroll
    for (int kk = 0; kk < kOrderKeys; ++kk) {
      const uint64_t bal = __ballot(k == kk);
      if (l == 0) wcnt_s[w * kOrderKeys + kk] = __popcll(bal);
      if (k == kk) rank = __popcll(bal & below);
    }
    __syncthreads();
    if (k >= 0) {
      int pos = rank;
#pragma unroll
      for (int kk = 0; kk < kOrderKeys; ++kk)
        if (kk == k) {
          pos += start[kk];
          for (int ww = 0; ww < w; ++ww) pos += wcnt_s[ww * kOrderKeys + kk];
        }
      a.order[pos] = L;
    }
#pragma unroll
    for (int kk = 0; kk < kOrderKeys; ++kk)
      for (int ww = 0; ww < kWaves; ++ww) start[kk] += wcnt_s[ww * kOrderKeys + kk];
    __syncthreads();
  }
}

// Q | K | V = X W^T + b for rows (b, i) of the padded batch; rows of padded
// nodes and the slots i in [n, NP) are written as zeros. Q, K: [B, H, NP, DH];
// V transposed: [B, H, DH, NP]. One block computes a 64-row x 64-feature tile:
// X and W chunks are staged in LDS with coalesced 16-byte loads, each wave
// computes 32 x 32 with MFMA, and the tile leaves through LDS so that every
// global store writes 16 contiguous bytes.
template <typename T, int D, int DH>
__global__ __launch_bounds__(kThreads) void qkv_kernel(LayerArgs a) {
  constexpr int H = D / DH;
  constexpr int KC = D < 128 ? D : 128;          // contraction chunk staged in LDS
  constexpr int NKC = D / KC;                    // chunks, all loaded before the first is used
  constexpr int EPC = 16 / (int)sizeof(T);       // elements per 16-byte chunk
  constexpr int CPR = KC / EPC;                  // chunks per staged row
  constexpr int PITCH = KC + 16 / (int)sizeof(T);  // padded LDS row pitch (elements)
  constexpr int OPITCH = 64 + 4;                 // output tile pitch (floats)
  static_assert(2 * 64 * PITCH * (int)sizeof(T) >= 64 * OPITCH * 4, "output tile fits");
  __shared__ __align__(16) T lds[2 * 64 * PITCH];
  T* xs = lds;
  T* wsm = lds + 64 * PITCH;

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, li = l & 15, lg = l >> 4;
  const uint32_t NP = a.NP, n = a.n;
  const uint32_t rows = (uint32_t)a.B * NP;  // < 2^31 (checked at context creation)
  const uint32_t m0 = blockIdx.x * 64u;
  // with a work order to write, column 0 is an extra column whose first
  // block (the first one dispatched) writes it
  const int yb = a.order ? (int)blockIdx.y - 1 : (int)blockIdx.y;
  if (yb < 0) {
    static_assert(sizeof(lds) >= kOrderMax + 128, "LDS of the work order");
    if (blockIdx.x == 0) work_order(a, reinterpret_cast<unsigned char*>(lds));
    return;
  }
  const int f0 = yb * 64;
  if (f0 >= 3 * D) {  // extra column of blocks
    global_film<T, H>(a, m0, 64u, rows);
    return;
  }
  const int which = f0 / D, fl0 = f0 % D;
  const T* W = static_cast<const T*>(which == 0 ? a.w_q : which == 1 ? a.w_k : a.w_v);
  const void* bias = which == 0 ? a.b_q : which == 1 ? a.b_k : a.b_v;
  const int wm = w & 1, wn = w >> 1;  // this wave's 32 x 32 quadrant

  f32x4 acc[2][2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Rows (b, i) of the tile without a division per row: NP >= 16, so a row
  // offset below 64 crosses at most four graph boundaries.
  const uint32_t b0 = m0 / NP, i00 = m0 - b0 * NP;
  auto split = [&](uint32_t off, uint32_t& b, uint32_t& i) {
    b = b0;
    i = i00 + off;
    while (i >= NP) { i -= NP; ++b; }
  };
  // The rows this thread stages: X rows are read whenever they exist (i < n)
  // and zeroed afterwards for padded nodes, so no load waits on the mask.
  constexpr int RPT = 64 * CPR / kThreads;  // staged chunks per thread and matrix
  static_assert((64 * CPR) % kThreads == 0, "staging split");
  float bcol[2];  // bias of this lane's output columns
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) bcol[nt] = ld_or0<T>(bias, fl0 + wn * 32 + nt * 16 + li);
  // Slots without a node read node 0 (a valid address) and are zeroed.
  const T* xsrc[RPT];
  const uint8_t* xmask[RPT];
  bool xexists[RPT];
#pragma unroll
  for (int k = 0; k < RPT; ++k) {
    const int row = (tid + k * kThreads) / CPR;
    uint32_t b, i;
    split(row, b, i);
    xexists[k] = m0 + row < rows && i < n;
    const size_t node = xexists[k] ? (size_t)b * n + i : 0;
    xsrc[k] = static_cast<const T*>(a.X) + node * D;
    xmask[k] = a.mask + node;
  }
  u32x4 xv[NKC][RPT], wv[NKC][RPT];
#pragma unroll
  for (int q = 0; q < NKC; ++q)
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
      const int idx = tid + k * kThreads, row = idx / CPR, ch = idx % CPR;
      xv[q][k] = *reinterpret_cast<const u32x4*>(xsrc[k] + q * KC + ch * EPC);
      wv[q][k] = *reinterpret_cast<const u32x4*>(W + (size_t)(fl0 + row) * D + q * KC + ch * EPC);
    }
  // mask bytes after the X and W loads, so waiting for them costs nothing extra
  bool xok[RPT];
#pragma unroll
  for (int k = 0; k < RPT; ++k) {
    const uint8_t mv = *xmask[k];
    xok[k] = xexists[k] && mv != 0;
  }
  bool rok[2][4];  // output rows of this lane that belong to real nodes
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t off = wm * 32 + mt * 16 + 4 * lg + r;
      uint32_t b, i;
      split(off, b, i);
      const bool exists = m0 + off < rows && i < n;
      const uint8_t mv = a.mask[exists ? (size_t)b * n + i : 0];
      rok[mt][r] = exists && mv != 0;
    }

#pragma unroll
  for (int q = 0; q < NKC; ++q) {
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
      const int idx = tid + k * kThreads, row = idx / CPR, ch = idx % CPR;
      *reinterpret_cast<u32x4*>(xs + row * PITCH + ch * EPC) = xok[k] ? xv[q][k] : u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(wsm + row * PITCH + ch * EPC) = wv[q][k];
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < KC / (4 * EPC); ++ks) {
      // lane group lg takes elements [ks*4*EPC + lg*EPC, +EPC) of the chunk
      Frag<T, EPC> af[2], bfr[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        af[t].load(xs + (wm * 32 + t * 16 + li) * PITCH + ks * 4 * EPC + lg * EPC);
        bfr[t].load(wsm + (wn * 32 + t * 16 + li) * PITCH + ks * 4 * EPC + lg * EPC);
      }
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = mma(acc[mt][nt], af[mt], bfr[nt]);
    }
    __syncthreads();
  }

  // epilogue: bias, padding rows to zero, tile through LDS as floats
  float* os = reinterpret_cast<float*>(lds);
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = wm * 32 + mt * 16 + 4 * lg + r;
      const bool ok = rok[mt][r];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int col = wn * 32 + nt * 16 + li;
        os[row * OPITCH + col] = ok ? acc[mt][nt][r] + bcol[nt] : 0.f;
      }
    }
  }
  __syncthreads();
  // 8 consecutive elements per thread and store
  for (int idx = tid; idx < 64 * 8; idx += kThreads) {
    if (which < 2) {
      const int row = idx >> 3, c8 = (idx & 7) * 8;  // 8 features of one row
      if (m0 + row >= rows) continue;
      uint32_t b, i;
      split(row, b, i);
      const int f = fl0 + c8, h = f / DH, t = f % DH;
      float v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = os[row * OPITCH + c8 + k];
      Frag<T, 8> o;
      o.set(v);
      o.store(static_cast<T*>(which == 0 ? a.Qw : a.Kw) + (((size_t)b * H + h) * NP + i) * DH + t);
    } else {
      const int col = idx >> 3, r8 = (idx & 7) * 8;  // 8 consecutive rows of one feature
      if (m0 + r8 >= rows) continue;
      uint32_t b, i;
      split(r8, b, i);
      const int f = fl0 + col, h = f / DH, t = f % DH;
      float v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = os[(r8 + k) * OPITCH + col];
      Frag<T, 8> o;
      o.set(v);
      o.store(static_cast<T*>(a.Vt) + (((size_t)b * H + h) * DH + t) * NP + i);
    }
  }
}

// ------------------------------------------------------------------ score stage

// E fragments of one 16 x 16 (query, key) tile: lane (li, lg) holds channels
// [lg*DE/4, (lg+1)*DE/4) of edge (i0 + li, j0 + jj) for jj = 0..15. Pairs
// that are not real (query or key masked, or past n) are not read: zeros.
template <typename T, int DE>
struct ETile {
  Frag<T, DE / 4> f[16];
  // Every pair, masked or not, with no mask bytes needed and no condition on
  // any load; pairs outside the n x n layout read the nearest pair inside it.
  // Values of pairs that are not real are discarded by the selects of the
  // score stage and of the edge update.
  // NT: with the non-temporal policy (E read once by the fused layer).
  template <bool NT = false>
  __device__ __forceinline__ void load_all(const T* E, int b, int n, int i, int j0, int lg) {
    const T* row = E + ((size_t)b * n + (i < n ? i : n - 1)) * n * DE + lg * (DE / 4);
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) {
      const int j = j0 + jj < n ? j0 + jj : n - 1;
      if constexpr (NT)
        f[jj].load_nt(row + (size_t)j * DE);
      else
        f[jj].load(row + (size_t)j * DE);
    }
  }
  __device__ __forceinline__ void load(const T* E, int b, int n, int i, bool mi, int j0, int lg, uint32_t bits) {
    const T* row = E + ((size_t)b * n + i) * n * DE + lg * (DE / 4);
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) {
      if (mi && ((bits >> jj) & 1u))
        f[jj].load(row + (size_t)(j0 + jj) * DE);
      else
        f[jj].zero();
    }
  }
};

// Per-lane state of one (graph b, 16-query block) for the score stage.
template <typename T, int H, int DH, int DE>
struct Scorer {
  int b, n, NP, JT, i, li, lg;
  bool mi;
  bool mi_any;  // some query of the block is real
  const uint8_t* mask_b;
  const T* E;
  const T* Kw;
  const T* Vt;
  float scale;
  Frag<T, DH / 4> qf[H];
  Frag<T, DE / 4> wf;  // edge-FiLM weights, row li: gamma of head li, then beta of head li-H
  Frag<T, 4> fb;       // FiLM biases of rows 4*lg .. 4*lg+3 (b_emul or b_eadd, or zeros)
  float gy[2 * H];     // gamma_y then beta_y of graph b

  // Per-lane constants; no loads.
  __device__ __forceinline__ void setup(const LayerArgs& a, int b_, int i0) {
    const int l = threadIdx.x & 63;
    li = l & 15; lg = l >> 4;
    b = b_; n = a.n; NP = a.NP; JT = a.NP / 16; i = i0 + li;
    mask_b = a.mask + (size_t)b * n;
    E = static_cast<const T*>(a.E);
    Kw = static_cast<const T*>(a.Kw);
    Vt = static_cast<const T*>(a.Vt);
    scale = a.scale;
  }
  // Mask bytes; slots past n read node n-1 and count as masked.
  __device__ __forceinline__ uint32_t query_mask_byte() const {
    const uint32_t v = mask_b[i < n ? i : n - 1];
    return i < n ? v : 0u;
  }
  __device__ __forceinline__ uint32_t key_mask_byte(int jt) const {
    const int j = 16 * jt + li;
    const uint32_t v = mask_b[j < n ? j : n - 1];
    return j < n ? v : 0u;
  }
  // Queries, FiLM weights and biases, global FiLM coefficients.
  __device__ __forceinline__ void load_weights(const LayerArgs& a) {
    load_film(a);
    load_queries(a);
  }
  // Edge-FiLM weights and biases (all the score stage needs besides E).
  // Without the per-edge FiLM (light-edge and no-score-modulation variants)
  // the weights and biases are zeros: gamma_e = 1 and beta_e = 0 exactly.
  __device__ __forceinline__ void load_film(const LayerArgs& a) {
    const bool ef = (a.variant & (kLightEdge | kNoScoreMod)) == 0;  // uniform
    const T* wrow = li < H ? static_cast<const T*>(a.w_emul) + (size_t)li * DE
                  : static_cast<const T*>(a.w_eadd) + (size_t)(li - H) * DE;
    wf.load(ef && li < 2 * H ? wrow + lg * (DE / 4) : zeros<T>());
    // FiLM rows 4*lg .. 4*lg+3 are all gamma rows or all beta rows (4 | H)
    static_assert(H % 4 == 0, "heads");
    const int r0 = 4 * lg;
    fb.load(r0 < H ? elem_or_zero<T>(a.b_emul, r0, ef) : elem_or_zero<T>(a.b_eadd, r0 - H, ef && r0 < 2 * H));
  }
  // Query fragments and the graph's global FiLM coefficients.
  __device__ __forceinline__ void load_queries(const LayerArgs& a) {
    const T* Qw = static_cast<const T*>(a.Qw);
#pragma unroll
    for (int h = 0; h < H; ++h) qf[h].load(Qw + (((size_t)b * H + h) * NP + i) * DH + lg * (DH / 4));
#pragma unroll
    for (int o = 0; o < 2 * H; ++o) gy[o] = a.gy[(size_t)b * 2 * H + o];
  }

  // K and V fragments of key tile jt. A tile past the padded size reads tile
  // JT-1 instead: its keys are masked (all logits -inf, all A exactly 0), and
  // workspace K and V values are finite, so they add nothing.
  __device__ __forceinline__ void load_k(int jt, Frag<T, DH / 4> (&kf)[H]) const {
    const int jc = jt < JT ? jt : JT - 1;
#pragma unroll
    for (int h = 0; h < H; ++h) kf[h].load(Kw + (((size_t)b * H + h) * NP + 16 * jc + li) * DH + lg * (DH / 4));
  }
  __device__ __forceinline__ void load_v(int jt, Frag<T, 4> (&vf)[H][DH / 16]) const {
    const int jc = jt < JT ? jt : JT - 1;
#pragma unroll
    for (int h = 0; h < H; ++h)
#pragma unroll
      for (int tc = 0; tc < DH / 16; ++tc)
        vf[h][tc].load(Vt + (((size_t)b * H + h) * DH + tc * 16 + li) * NP + 16 * jc + 4 * lg);
  }

  // Masked logits u[h][r] of query i for key j = 16*jt + 4*lg + r from the
  // tile's E fragments and K fragments; bits: real keys of the tile.
  // SKIP_EMPTY: a tile without real keys returns early (a branch that lets
  // the compiler sink the loads it guards behind the mask bytes).
  template <bool SKIP_EMPTY = true>
  __device__ __forceinline__ void logits(const ETile<T, DE>& et, const Frag<T, DH / 4> (&kf)[H], uint32_t bits,
                                         float (&u)[H][4]) const {
    if (SKIP_EMPTY && bits == 0u) {
      no_keys(u);
      return;
    }
    const f32x4 fc = film_start();
    float R[4][16];  // R[x][4*r' + r]: key 4*x + r', film row 4*lg + r
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) film(et.f[jj], fc, R, jj);
    scores(R, kf, bits, u);
  }

  // The same for float32 data, whose E tile would not fit in registers next
  // to the rest: the fragments of key tile j0 are read here in groups of 2
  // keys, the next group in flight while the current one is used.
  __device__ __forceinline__ void logits_streamed(int j0, const Frag<T, DH / 4> (&kf)[H], uint32_t bits,
                                                  float (&u)[H][4]) const {
    constexpr int G = 2, NG = 16 / G;
    if (bits == 0u) {
      no_keys(u);
      return;
    }
    const T* row = E + ((size_t)b * n + i) * n * DE + lg * (DE / 4);
    const f32x4 fc = film_start();
    float R[4][16];
    Frag<T, DE / 4> eg[2][G];
    auto load_group = [&](Frag<T, DE / 4>(&f)[G], int g) {
#pragma unroll
      for (int q = 0; q < G; ++q) {
        const int jj = G * g + q;
        if (mi && ((bits >> jj) & 1u)) f[q].load(row + (size_t)(j0 + jj) * DE);
        else f[q].zero();
      }
    };
    load_group(eg[0], 0);
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      if (g + 1 < NG) load_group(eg[(g + 1) & 1], g + 1);
      __builtin_amdgcn_sched_barrier(0);  // no more than two groups live
#pragma unroll
      for (int q = 0; q < G; ++q) film(eg[g & 1][q], fc, R, G * g + q);
      __builtin_amdgcn_sched_barrier(0);
    }
    scores(R, kf, bits, u);
  }

  __device__ __forceinline__ static void no_keys(float (&u)[H][4]) {
#pragma unroll
    for (int h = 0; h < H; ++h)
#pragma unroll
      for (int r = 0; r < 4; ++r) u[h][r] = kNegInf;
  }
  // Edge FiLM on MFMA: column = query row, rows = (gamma, beta) x head; the
  // accumulator starts at 1 + b_emul (gamma rows) or b_eadd (beta rows).
  __device__ __forceinline__ f32x4 film_start() const {
    f32x4 fc;
#pragma unroll
    for (int r = 0; r < 4; ++r) fc[r] = (4 * lg < H ? 1.f : 0.f) + fb.get(r);
    return fc;
  }
  __device__ __forceinline__ void film(const Frag<T, DE / 4>& e, const f32x4& fc, float (&R)[4][16], int jj) const {
    const f32x4 F = mma(fc, wf, e);
#pragma unroll
    for (int r = 0; r < 4; ++r) R[jj >> 2][4 * (jj & 3) + r] = F[r];
  }
  // From the FiLM rows of the 16 keys to the masked logits.
  __device__ __forceinline__ void scores(float (&R)[4][16], const Frag<T, DH / 4> (&kf)[H], uint32_t bits,
                                         float (&u)[H][4]) const {
    f32x4 S[H];
    qk(kf, S);
    scores_from(R, S, bits, u);
  }
  // S^T = K Q^T per head: lane (li, lg) gets query i0 + li, keys 4*lg + r.
  __device__ __forceinline__ void qk(const Frag<T, DH / 4> (&kf)[H], f32x4 (&S)[H]) const {
#pragma unroll
    for (int h = 0; h < H; ++h) S[h] = mma(f32x4{0.f, 0.f, 0.f, 0.f}, kf[h], qf[h]);
  }
  __device__ __forceinline__ void scores_from(float (&R)[4][16], const f32x4 (&S)[H], uint32_t bits,
                                              float (&u)[H][4]) const {
    // now R[x][4*r' + r]: key 4*lg + r', film row 4*x + r
    lane_group_transpose<16>(R);
    // real pairs of this lane (bit r: key 4*lg + r), as plain bit tests: a
    // short-circuit condition here becomes divergent branches around the
    // whole logit array
    const uint32_t okb = (bits >> (4 * lg)) & (mi ? 0xfu : 0u);
#pragma unroll
    for (int h = 0; h < H; ++h) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float gam = R[h >> 2][4 * r + (h & 3)];
        const float bet = R[(H + h) >> 2][4 * r + ((H + h) & 3)];
        const float v = ((S[h][r] * scale) * gam + bet) * gy[h] + gy[H + h];
        u[h][r] = ((okb >> r) & 1u) ? v : kNegInf;
      }
    }
  }
};

// E streamed through LDS in half tiles (bfloat16, de = 64): the 8 keys of one
// half of a 16 x 16 (query, key) tile. LDS row r holds query row i0 + r: its
// 8 keys, 1 KB contiguous in E, padded by 16 bytes so that the fragment reads
// below fall on distinct banks.
template <typename T, int DE>
struct EHalf {
  static_assert(sizeof(T) == 2 && DE == 64, "bfloat16, de = 64");
  static constexpr int kRowPitch = 8 * DE * 2 + 16;  // bytes
  static constexpr int kBytes = 16 * kRowPitch;      // one half tile
  // 16 global-to-LDS loads, one per query row, into half `half` of the two
  // half tiles at ebase: lane l moves the 16-byte piece l % 8 of key
  // 16 jt + 8 half + l / 8. Rows and keys past n read row and key n - 1
  // (their values are discarded by the selects of the score stage and of the
  // edge update).
  template <int CPOL = kCpolDefault>
  static __device__ __forceinline__ void fetch(const T* Eb, int n, int i0, int jt, int half, unsigned char* ebase,
                                               int l) {
    const int j = 16 * jt + 8 * half + (l >> 3);
    const int jc = j < n ? j : n - 1;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int ir = i0 + r < n ? i0 + r : n - 1;
      const T* src = Eb + ((size_t)ir * n + jc) * DE + (l & 7) * 8;
      __builtin_amdgcn_global_load_lds((const void*)src,
                                       (__attribute__((address_space(3))) void*)(ebase + half * kBytes + r * kRowPitch),
                                       16, 0, CPOL);
    }
  }
  // This lane's E fragments (query row li, channel quarter lg) of all 8 keys
  // of the half, read in one asm block that also waits for the reads. The
  // compiler cannot tell which LDS bytes a global-to-LDS transfer writes, so
  // before any LDS read it sees, it waits for every transfer in flight; reads
  // it does not see leave the next half tile in flight (the kernels wait for
  // the half tile they read explicitly).
  static __device__ __forceinline__ void frags8(const unsigned char* half, int li, int lg, Frag<T, DE / 4> (&e)[8]) {
    const uint32_t a = (uint32_t)(size_t)(__attribute__((address_space(3))) const unsigned char*)(
        half + li * kRowPitch + lg * (DE / 4) * 2);
    u32x4 v[16];
    asm volatile(
        "ds_read_b128 %0, %16\n\t"
        "ds_read_b128 %1, %16 offset:16\n\t"
        "ds_read_b128 %2, %16 offset:128\n\t"
        "ds_read_b128 %3, %16 offset:144\n\t"
        "ds_read_b128 %4, %16 offset:256\n\t"
        "ds_read_b128 %5, %16 offset:272\n\t"
        "ds_read_b128 %6, %16 offset:384\n\t"
        "ds_read_b128 %7, %16 offset:400\n\t"
        "ds_read_b128 %8, %16 offset:512\n\t"
        "ds_read_b128 %9, %16 offset:528\n\t"
        "ds_read_b128 %10, %16 offset:640\n\t"
        "ds_read_b128 %11, %16 offset:656\n\t"
        "ds_read_b128 %12, %16 offset:768\n\t"
        "ds_read_b128 %13, %16 offset:784\n\t"
        "ds_read_b128 %14, %16 offset:896\n\t"
        "ds_read_b128 %15, %16 offset:912\n\t"
        "s_waitcnt lgkmcnt(0)"
        // early-clobber outputs: a read may land before a later one has
        // taken its address from the input register
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]), "=&v"(v[7]),
          "=&v"(v[8]), "=&v"(v[9]), "=&v"(v[10]), "=&v"(v[11]), "=&v"(v[12]), "=&v"(v[13]), "=&v"(v[14]), "=&v"(v[15])
        : "v"(a));
    static_assert(DE * 2 == 128, "key pitch of the offsets above");
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      e[k].w[0] = v[2 * k].x; e[k].w[1] = v[2 * k].y; e[k].w[2] = v[2 * k].z; e[k].w[3] = v[2 * k].w;
      e[k].w[4] = v[2 * k + 1].x; e[k].w[5] = v[2 * k + 1].y; e[k].w[6] = v[2 * k + 1].z; e[k].w[7] = v[2 * k + 1].w;
    }
  }
  // This lane's E fragment (query row li, channel quarter lg) of key k of the
  // half: two 16-byte LDS reads.
  static __device__ __forceinline__ Frag<T, DE / 4> frag(const unsigned char* half, int li, int lg, int k) {
    const unsigned char* p = half + li * kRowPitch + lg * (DE / 4) * 2 + k * DE * 2;
    const u32x4 v0 = *reinterpret_cast<const u32x4*>(p);
    const u32x4 v1 = *reinterpret_cast<const u32x4*>(p + 16);
    Frag<T, DE / 4> e;
    e.w[0] = v0.x; e.w[1] = v0.y; e.w[2] = v0.z; e.w[3] = v0.w;
    e.w[4] = v1.x; e.w[5] = v1.y; e.w[6] = v1.z; e.w[7] = v1.w;
    return e;
  }
};

// +0.0 into the edge outputs of one 16 x 16 tile (pairs inside the n x n layout).
template <typename T, int DE>
__device__ __forceinline__ void zero_edge_tile(T* Eout, int b, int n, int i, int j0, int lg) {
  if (i >= n) return;
  T* row = Eout + ((size_t)b * n + i) * n * DE + lg * (DE / 4);
  Frag<T, DE / 4> z;
  z.zero();
#pragma unroll
  for (int jj = 0; jj < 16; ++jj)
    if (j0 + jj < n) z.store(row + (size_t)(j0 + jj) * DE);
}

// ------------------------------------------------------------------ edge update

// Residual edge update of one 16 x 16 (query, key) tile. Per key j and
// 16-channel chunk: E'^T (channels x queries) = W_e (channels x heads) A^T
// + E^T (+ b_e), with A given as this lane's values for keys 4*lg + r and all
// heads; they are regrouped in registers so that lane group lg supplies heads
// [lg*QH, (lg+1)*QH) for every key. In bfloat16 mode the contraction has 16
// slots for H <= 12 heads; slot H carries 1 against b_e, and E^T enters
// through a second MFMA against the identity (exact: products by 1 and sums
// with zeros), straight from its packed fragment, so the update spends no
// VALU work on E.
template <typename T, int H, int DE>
struct Updater {
  static constexpr bool kBF = sizeof(T) == 2;
  static constexpr int QH = kBF ? 4 : H / 4;  // heads per lane group
  static constexpr int NCH = DE / 16;
  static constexpr int RW = kBF ? 8 : 4 * QH;  // 32-bit words per key group of the head operand
  Frag<T, QH> wef[NCH];
  Frag<T, 4> eye;                    // identity rows li, slots 4*lg .. 4*lg+3 (bfloat16)
  T bl[kBF ? NCH : 1];               // raw b_e values of the bias lane group (bfloat16)
  Frag<T, kBF ? 4 : DE / 4> bfr;     // raw b_e of this lane's channels (fp32)
  bool has_heads, bias_lane;

  // Issues the loads only; finish() builds the operands once they are needed.
  __device__ __forceinline__ void init(const LayerArgs& a, int li, int lg) {
    const T* We = static_cast<const T*>(a.w_e);
    has_heads = lg * QH < H || (kBF && lg * QH == H && a.b_e);
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
      // MFMA row li of chunk ch is channel (li/4)*(DE/4) + 4*ch + li%4, so that
      // output rows 4*lg + r land on this lane group's channel quarter.
      const int c = (li >> 2) * (DE / 4) + 4 * ch + (li & 3);
      wef[ch].load(lg * QH < H ? We + (size_t)c * H + lg * QH : zeros<T>());
      // lane group H / QH: b_e goes in slot 0, against the constant-1 head slot
      if constexpr (kBF) bl[ch] = *elem_or_zero<T>(a.b_e, c, lg * QH == H);
    }
    bias_lane = kBF && lg * QH == H;
    if constexpr (kBF) {
      constexpr uint32_t kOne = 0x3f80u;  // bfloat16 1.0
      const int q = li - 4 * lg;         // slot of the diagonal in this lane, if any
      eye.w[0] = (q == 0 ? kOne : 0u) | (q == 1 ? kOne << 16 : 0u);
      eye.w[1] = (q == 2 ? kOne : 0u) | (q == 3 ? kOne << 16 : 0u);
    } else {
      bfr.load(elem_or_zero<T>(a.b_e, lg * (DE / 4), true));
    }
  }
  __device__ __forceinline__ void finish() {
    if constexpr (kBF) {
#pragma unroll
      for (int ch = 0; ch < NCH; ++ch)  // slot 0 is the low half of dword 0
        wef[ch].w[0] = bias_lane ? (uint32_t)bl[ch] : wef[ch].w[0];
    }
  }

  // KEEP: et holds the tile's E fragments; otherwise E is read here.
  // bits: real keys of the tile; full: every pair of the tile is real.
  // A: this lane's attention values in the storage type, keys 4*lg .. 4*lg+3
  // of each head (the layout of the A store and of the A V operand).
  // mid() runs once, after the first 8 keys (every caller's wave must reach
  // it exactly once: it may hold a barrier).
  // The head operand of the update's products for one tile, from A as laid
  // out by the A store (this lane: keys 4*lg .. 4*lg+3 of each head);
  // afterwards block x of lane group lg holds key 4*x + r', heads
  // lg*QH .. (lg+1)*QH - 1.
  __device__ __forceinline__ void head_operand(const Frag<T, 4> (&A)[H], float (&R)[4][RW]) const {
    if constexpr (kBF) {
      // R[x][2*r' + q2]: packed bfloat16 pair (head 4x + 2q2, head 4x + 2q2 + 1)
      // of key 4*lg + r'; slot H holds 1 (against b_e), the rest 0
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int rp = 0; rp < 4; ++rp)
#pragma unroll
          for (int q2 = 0; q2 < 2; ++q2) {
            const int h0 = 4 * x + 2 * q2;
            uint32_t v = h0 == H ? 0x3f80u : 0u;  // bfloat16 1.0 in the low half
            if (h0 < H)  // H is even: key r' of heads h0 and h0 + 1, taken from their key pairs
              v = __builtin_amdgcn_perm(A[h0 + 1].w[rp >> 1], A[h0].w[rp >> 1], (rp & 1) ? 0x07060302u : 0x05040100u);
            R[x][2 * rp + q2] = __uint_as_float(v);
          }
    } else {
      // R[x][r'*QH + q]: key 4*lg + r', head x*QH + q
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int rp = 0; rp < 4; ++rp)
#pragma unroll
          for (int q = 0; q < QH; ++q) {
            const int h = x * QH + q;
            R[x][rp * QH + q] = h < H ? A[h].get(rp) : 0.f;
          }
    }
    lane_group_transpose<RW>(R);
  }

  template <bool KEEP, typename Mid>
  __device__ __forceinline__ void tile(const ETile<T, DE>& et, const T* E, T* Eout, int b, int n, int i,
                                       bool mi, int j0, int lg, uint32_t bits, bool full,
                                       const Frag<T, 4> (&A)[H], Mid&& mid) const {
    float R[4][RW];
    head_operand(A, R);
    const size_t rowoff = ((size_t)b * n + i) * n * DE + lg * (DE / 4);
    if (bits == 0u) {  // no real pair in the tile (uniform): zeros only
      zero_edge_tile<T, DE>(Eout, b, n, i, j0, lg);
      mid();
      return;
    }
    const uint32_t okj = mi ? bits : 0u;  // bit jj: pair (i, j0 + jj) is real
    const bool iin = i < n;
    if constexpr (KEEP) {
      if (full) {
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
          if (jj == 8) mid();
          step<true>(et.f[jj], Eout, rowoff + (size_t)(j0 + jj) * DE, true, true, R, jj);
        }
      } else {
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
          if (jj == 8) mid();
          step<false>(et.f[jj], Eout, rowoff + (size_t)(j0 + jj) * DE, iin & (j0 + jj < n), (okj >> jj) & 1u, R, jj);
        }
      }
    } else if constexpr (kBF) {
      // E read again, kPf keys ahead of their use. The loads are
      // unconditional (pairs outside the n x n map read the zero table), so
      // they stay in flight across keys; values of masked pairs are
      // discarded by the step's select.
      constexpr int kPf = 4;
      Frag<T, DE / 4> buf[kPf];
      auto src = [&](int jj) {
        return (iin && j0 + jj < n) ? E + rowoff + (size_t)(j0 + jj) * DE : zeros<T>();
      };
#pragma unroll
      for (int q = 0; q < kPf; ++q) buf[q].load(src(q));
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) {
        if (jj == 8) mid();
        const size_t off = rowoff + (size_t)(j0 + jj) * DE;
        const Frag<T, DE / 4> ef = buf[jj % kPf];
        if (jj + kPf < 16) buf[jj % kPf].load(src(jj + kPf));
        step<false>(ef, Eout, off, iin & (j0 + jj < n), (okj >> jj) & 1u, R, jj);
      }
    } else {
      // float32: E read in groups of 4 keys, the next group in flight (the
      // whole tile would not fit in registers next to the rest)
      Frag<T, DE / 4> eg[2][4];
      auto load_group = [&](Frag<T, DE / 4>(&f)[4], int g) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int jj = 4 * g + q;
          if ((okj >> jj) & 1u) f[q].load(E + rowoff + (size_t)(j0 + jj) * DE);
          else f[q].zero();
        }
      };
      load_group(eg[0], 0);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        if (g == 2) mid();
        if (g < 3) load_group(eg[(g + 1) & 1], g + 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int jj = 4 * g + q;
          step<false>(eg[g & 1][q], Eout, rowoff + (size_t)(j0 + jj) * DE, iin & (j0 + jj < n), (okj >> jj) & 1u, R, jj);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // The outputs of one key of the tile: ef holds this lane's E channels of
  // pair (i, j); masked pairs give +0.0 (unless FULL: every pair is real).
  template <bool FULL>
  __device__ __forceinline__ void outputs(const Frag<T, DE / 4>& ef, bool real, const float (&R)[4][RW], int jj,
                                          float (&out)[DE / 4]) const {
    Frag<T, QH> af;
    if constexpr (kBF) {
      af.w[0] = has_heads ? __float_as_uint(R[jj >> 2][2 * (jj & 3)]) : 0u;
      af.w[1] = has_heads ? __float_as_uint(R[jj >> 2][2 * (jj & 3) + 1]) : 0u;
    } else {
      if (has_heads) af.set(&R[jj >> 2][(jj & 3) * QH]); else af.zero();
    }
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
      f32x4 c;
      if constexpr (kBF) {
        // channels 4*ch .. 4*ch+3 of this lane's quarter are dwords 2*ch, 2*ch+1
        Frag<T, 4> e4;
        e4.w[0] = ef.w[2 * ch];
        e4.w[1] = ef.w[2 * ch + 1];
        c = mma(f32x4{0.f, 0.f, 0.f, 0.f}, eye, e4);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) c[r] = ef.get(4 * ch + r) + bfr.get(4 * ch + r);
      }
      c = mma(c, wef[ch], af);
#pragma unroll
      for (int r = 0; r < 4; ++r) out[4 * ch + r] = (FULL || real) ? c[r] : 0.f;
    }
  }
  // One key of the tile, stored when the pair lies inside the layout (inb).
  template <bool FULL>
  __device__ __forceinline__ void step(const Frag<T, DE / 4>& ef, T* Eout, size_t off, bool inb, bool real,
                                       const float (&R)[4][RW], int jj) const {
    float out[DE / 4];
    outputs<FULL>(ef, real, R, jj, out);
    if (FULL || inb) {
      Frag<T, DE / 4> of;
      of.set(out);
      of.store(Eout + off);
    }
  }
  // One key of the tile, stored by every lane to dst (the caller points lanes
  // whose pair lies outside the layout at a sink).
  template <bool FULL>
  __device__ __forceinline__ void step_to(const Frag<T, DE / 4>& ef, T* dst, bool real, const float (&R)[4][RW],
                                          int jj) const {
    float out[DE / 4];
    outputs<FULL>(ef, real, R, jj, out);
    Frag<T, DE / 4> of;
    of.set(out);
    of.store(dst);
  }
};

// Row pitch (floats) of the O partials in LDS: 4 floats of padding put the
// 16-byte writes of 8 consecutive query rows on distinct banks.
template <int D>
constexpr int kOPitch = D + 4;

// Cross-wave reduction of the per-wave O^T partials and the store of O rows.
// Lane (li, lg) holds O[i0 + li][h*DH + 16*tc + 4*lg + r] in oacc[h][tc][r]:
// 4 consecutive channels, written to LDS as one 16-byte row piece.
template <int H, int DH>
__device__ __forceinline__ void o_partials_to_lds(float* os, const f32x4 (&oacc)[H][DH / 16], int w, int li, int lg) {
  constexpr int D = H * DH, OP = kOPitch<D>;
#pragma unroll
  for (int h = 0; h < H; ++h)
#pragma unroll
    for (int tc = 0; tc < DH / 16; ++tc)
      *reinterpret_cast<f32x4*>(os + (w * 16 + li) * OP + h * DH + tc * 16 + 4 * lg) = oacc[h][tc];
}
// After a barrier that follows every wave's o_partials_to_lds.
template <typename T, int H, int DH>
__device__ __forceinline__ void o_reduce_store(const LayerArgs& a, const float* os, int b, int i0, uint32_t qbits) {
  constexpr int D = H * DH, OP = kOPitch<D>;
  for (int idx = threadIdx.x; idx < 16 * D / 4; idx += kThreads) {
    const int il = idx / (D / 4), c = (idx % (D / 4)) * 4, ii = i0 + il;
    if (ii >= a.n) continue;
    f32x4 s = *reinterpret_cast<const f32x4*>(os + il * OP + c);
#pragma unroll
    for (int ww = 1; ww < kWaves; ++ww) s += *reinterpret_cast<const f32x4*>(os + (ww * 16 + il) * OP + c);
    const bool real = (qbits >> il) & 1u;
    float v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = real ? s[k] : 0.f;
    Frag<T, 4> o;
    o.set(v);
    o.store(static_cast<T*>(a.O) + ((size_t)b * a.n + ii) * D + c);
  }
}
template <typename T, int H, int DH>
__device__ __forceinline__ void reduce_store_O(const LayerArgs& a, float* os, const f32x4 (&oacc)[H][DH / 16],
                                               int b, int i0, int w, int li, int lg, uint32_t qbits) {
  o_partials_to_lds<H, DH>(os, oacc, w, li, lg);
  __syncthreads();
  o_reduce_store<T, H, DH>(a, os, b, i0, qbits);
}

// Whether all 16 queries of the block and all 16 keys of the tile are real.
__device__ __forceinline__ bool tile_full(bool mi, uint32_t bits) {
  return bits == 0xffffu && (__ballot(mi) & 0xffffull) == 0xffffull;
}

// Wait until at most N vector memory operations of this wave are in flight
// (s_waitcnt with vmcnt N and the other counters at their maximum). The
// counter retires operations in issue order.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x3 << 14)); }
// Barrier for data exchanged through LDS only: this wave's LDS operations are
// complete before s_barrier, and its global memory operations stay in
// flight (__syncthreads() waits for those as well). The empty asm statements
// keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  __asm__ __volatile__("" ::: "memory");
  wait_lgkmcnt0();
  __builtin_amdgcn_s_barrier();
  __asm__ __volatile__("" ::: "memory");
}

// ------------------------------------------------------------------ attention

// A block without a real query: its rows of A, O (and E') are +0.0. Wave w
// writes the key tiles w, w + kWaves, ... of its rows.
template <typename T, int H, int DH, int DE, int MAXT, bool EDGE>
__device__ __forceinline__ void zero_block(const LayerArgs& a, int b, int i0, int i, int w, int lg) {
  constexpr int D = H * DH;
  const int n = a.n, JT = a.NP / 16;
  T* Ag = static_cast<T*>(a.A);
#pragma unroll
  for (int tt = 0; tt < MAXT; ++tt) {
    const int jt = w + kWaves * tt, jb = 16 * jt + 4 * lg;
    if (jt >= JT || i >= n) continue;
    Frag<T, 4> z;
    z.zero();
#pragma unroll
    for (int h = 0; h < H; ++h) {
      T* row = Ag + (((size_t)b * H + h) * n + i) * n;
      if ((n & 3) == 0) {  // uniform: 4 keys in or out together, one vector store
        if (jb < n) z.store(row + jb);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (jb + r < n) Num<T>::st(row + jb + r, 0.f);
      }
    }
    if constexpr (EDGE) zero_edge_tile<T, DE>(static_cast<T*>(a.E_out), b, n, i, 16 * jt, lg);
  }
  for (int idx = threadIdx.x; idx < 16 * D / 4; idx += kThreads) {
    const int il = idx / (D / 4), c = (idx % (D / 4)) * 4;
    if (i0 + il >= n) continue;
    Frag<T, 4> z;
    z.zero();
    z.store(static_cast<T*>(a.O) + ((size_t)b * n + i0 + il) * D + c);
  }
}

// Single-pass tail shared by kSingle and kFused: masked softmax over the full
// row (lane groups by register swaps, waves through LDS), A rounded to the
// storage type and stored, O^T += V^T A^T on MFMA, the residual edge update
// (kFused) and the cross-wave O reduction. With KEEP_E the tile's E fragments
// were kept in registers (E read once); otherwise the update reads E again.
template <typename T, int H, int DH, int DE, int MAXT, int MODE, bool KEEP_E>
__device__ __forceinline__ void attn_rest(const LayerArgs& a, const Scorer<T, H, DH, DE>& sc,
                                          float (&u)[MAXT][H][4], const uint32_t (&bits)[MAXT],
                                          Frag<T, 4> (&vf)[H][DH / 16], float* os_s,
                                          float (&red_s)[2][kWaves][H][16], const ETile<T, DE>& et,
                                          Updater<T, H, DE>& up) {
  const int w = threadIdx.x >> 6, li = sc.li, lg = sc.lg;
  const int b = sc.b, n = a.n, JT = sc.JT, i = sc.i, i0 = i - li;
  // several tiles: the first tile's V now (no wait in the softmax covers it),
  // each next one right after the previous A V, ahead of that tile's A stores
  if constexpr (MAXT > 1) sc.load_v(w, vf);
  f32x4 oacc[H][DH / 16];
#pragma unroll
  for (int h = 0; h < H; ++h)
#pragma unroll
    for (int tc = 0; tc < DH / 16; ++tc) oacc[h][tc] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int h = 0; h < H; ++h) {
    float m = kNegInf;
#pragma unroll
    for (int tt = 0; tt < MAXT; ++tt)
#pragma unroll
      for (int r = 0; r < 4; ++r) m = fmaxf(m, u[tt][h][r]);
    m = lg_max(m);
    if (lg == 0) red_s[0][w][h][li] = m;
  }
  __syncthreads();
  float inv[H];
#pragma unroll
  for (int h = 0; h < H; ++h) {
    float M = kNegInf;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, red_s[0][ww][h][li]);
    // exp(u - M) as 2^(u log2 e - M log2 e): one FMA and one v_exp_f32; masked
    // logits (-inf) give exactly 0, and a row without real keys takes M = 0
    const float mb = (M == kNegInf) ? 0.f : M * kLog2e;
    float s = 0.f;
#pragma unroll
    for (int tt = 0; tt < MAXT; ++tt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(u[tt][h][r], kLog2e, -mb));
        u[tt][h][r] = p;
        s += p;
      }
    s = lg_sum(s);
    if (lg == 0) red_s[1][w][h][li] = s;
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < H; ++h) {
    float L = 0.f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) L += red_s[1][ww][h][li];
    // 1 / L on the reciprocal unit (about 1 ulp; the quotient feeds a
    // bfloat16 or a 1e-4-relative float32 result)
    inv[h] = (L > 0.f) ? __builtin_amdgcn_rcpf(L) : 0.f;
  }
  T* Ag = static_cast<T*>(a.A);
  // A in the storage type, once: the same fragments are stored, feed A V and
  // feed the edge update
  Frag<T, 4> ak[MAXT][H];
#pragma unroll
  for (int tt = 0; tt < MAXT; ++tt) {
    const int jt = w + kWaves * tt, j0 = 16 * jt;
#pragma unroll
    for (int h = 0; h < H; ++h) {
      float p[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) p[r] = u[tt][h][r] * inv[h];
      ak[tt][h].set(p);
    }
    if (jt < JT) {
      const int jb = j0 + 4 * lg;
      if ((n & 3) == 0) {  // uniform: 4 keys in or out together, one vector store
        if (i < n && jb < n) {
#pragma unroll
          for (int h = 0; h < H; ++h) ak[tt][h].store(Ag + (((size_t)b * H + h) * n + i) * n + jb);
        }
      } else if (i < n) {
#pragma unroll
        for (int h = 0; h < H; ++h) {
          T* row = Ag + (((size_t)b * H + h) * n + i) * n;
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (jb + r < n) Num<T>::st(row + jb + r, ak[tt][h].get(r));
        }
      }
#pragma unroll
      for (int h = 0; h < H; ++h)
#pragma unroll
        for (int tc = 0; tc < DH / 16; ++tc) oacc[h][tc] = mma(oacc[h][tc], vf[h][tc], ak[tt][h]);
    }
    if constexpr (MAXT > 1)
      if (tt + 1 < MAXT) sc.load_v(w + kWaves * (tt + 1), vf);
  }
  const uint32_t qbits = (uint32_t)(__ballot(sc.mi) & 0xffffull);
  if constexpr (MODE == kFused) {
    // O's cross-wave reduction runs between the two halves of the first
    // tile's update, while the first half's E' stores drain
    o_partials_to_lds<H, DH>(os_s, oacc, w, li, lg);
    auto reduce_O = [&] {
      __syncthreads();
      o_reduce_store<T, H, DH>(a, os_s, b, i0, qbits);
    };
    auto nothing = [] {};
    up.finish();
#pragma unroll
    for (int tt = 0; tt < MAXT; ++tt) {
      const int jt = w + kWaves * tt;
      const bool full = tile_full(sc.mi, bits[tt]);
      if (tt == 0) {
        if (jt < JT)
          up.template tile<KEEP_E>(et, sc.E, static_cast<T*>(a.E_out), b, n, i, sc.mi, 16 * jt, lg, bits[tt], full,
                                   ak[tt], reduce_O);
        else
          reduce_O();
      } else if (jt < JT) {
        up.template tile<KEEP_E>(et, sc.E, static_cast<T*>(a.E_out), b, n, i, sc.mi, 16 * jt, lg, bits[tt], full,
                                 ak[tt], nothing);
      }
    }
  } else {
    reduce_store_O<T, H, DH>(a, os_s, oacc, b, i0, w, li, lg, qbits);
  }
}

// One block per (graph, 16-query block); wave w owns key tiles w, w+4, ... .
// kSingle/kFused/kLogits keep the MAXT logit tiles of a wave in registers
// (n <= 64*MAXT); kOnline streams any n. Loads are issued in the order they
// are consumed so that a wait never covers the E stream early: mask bytes,
// then queries, weights, K and V fragments, then the E tile. With one tile per
// wave and bfloat16 data the fused mode keeps the E fragments in registers
// from the scores to the edge update (E read once).
template <typename T, int H, int DH, int DE, int MAXT, int MODE>
__global__ __launch_bounds__(kThreads) void attn_kernel(LayerArgs a) {
  constexpr int D = H * DH;
  constexpr bool kKeepE = MODE == kFused && MAXT == 1 && sizeof(T) == 2;
  static_assert(D <= 256 && 2 * H <= 16, "shape");
  // Two-pass pass 1 in bfloat16 with de = 64 streams E through LDS (see the
  // kOnline branch); the O partials of the epilogue reuse that space once
  // every wave has left its key loop.
  constexpr bool kPipe = MODE == kOnline && sizeof(T) == 2 && DE == 64;
  constexpr int kRowPitch = 8 * DE * 2 + 16;            // bytes: 8 keys of one query row, padded
  constexpr int kHalfBytes = 16 * kRowPitch;            // 16 query rows
  constexpr int kOBytes = kWaves * 16 * kOPitch<D> * 4;
  constexpr int kEBytes = kPipe ? kWaves * 2 * kHalfBytes : 0;
  __shared__ __align__(16) unsigned char smem_raw[kOBytes > kEBytes ? kOBytes : kEBytes];
  float* os_s = reinterpret_cast<float*>(smem_raw);  // O partials of each wave
  __shared__ float red_s[2][kWaves][H][16];

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, li = l & 15, lg = l >> 4;
  int ib, b;
  xcd_block(ib, b);
  const int i0 = ib * 16;
  Scorer<T, H, DH, DE> sc;
  sc.setup(a, b, i0);
  const int JT = sc.JT, n = a.n, NP = a.NP, i = sc.i;

  if constexpr (MODE == kOnline) {
    const uint32_t mq = sc.query_mask_byte();
    uint32_t mk = kPipe ? 0u : sc.key_mask_byte(w);
    sc.load_weights(a);
    sc.mi = mq != 0u;
    sc.mi_any = (__ballot(sc.mi) & 0xffffull) != 0ull;
    f32x4 oacc[H][DH / 16];
#pragma unroll
    for (int h = 0; h < H; ++h)
#pragma unroll
      for (int tc = 0; tc < DH / 16; ++tc) oacc[h][tc] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run[H], l_run[H];
#pragma unroll
    for (int h = 0; h < H; ++h) { m_run[h] = kNegInf; l_run[h] = 0.f; }
    // online softmax step for one key tile with logits u and its V fragments
    auto online_step = [&](float (&u)[H][4], const Frag<T, 4> (&vf)[H][DH / 16]) {
#pragma unroll
      for (int h = 0; h < H; ++h) {
        const float tm = lg_max(fmaxf(fmaxf(u[h][0], u[h][1]), fmaxf(u[h][2], u[h][3])));
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
          oacc[h][tc] *= alpha;
          oacc[h][tc] = mma(oacc[h][tc], vf[h][tc], af);
        }
      }
    };
    if constexpr (kPipe) {
      // E through LDS in half tiles (8 keys). Each half tile of the wave's
      // next key tile is fetched by 16 global-to-LDS loads, one per query
      // row, each moving that row's 8 keys (1 KB, contiguous in E) into a
      // padded LDS row; the FiLM products read each key's fragment straight
      // from LDS (two 16-byte reads per lane, no bank conflicts), so the E
      // tile never sits in registers. A half is refetched as soon as this
      // tile's FiLM products have read it, so the next tile streams in while
      // this one's second half, scores, softmax and A V run. Per tile the
      // wave issues, in this order: half 0 (16 loads), half 1 (16), the key
      // mask byte (1), K (H), V (H DH / 16); every load is unconditional
      // (after the last tile they read the zero table or a clamped tile), so
      // the waits below count exactly. Every pair is read (masked values are
      // discarded by the selects of the score stage). The transfers take the
      // streaming cache policy, since pass 1 reads E once: over a loop of
      // layer calls at B = 4, n = 1024 pass 1 went from 141 to 112 us with
      // it and pass 2, which then finds none of E in the Infinity Cache,
      // from 206 to 224 us (the layer from 355 to 341 us).
      constexpr int kV = H * (DH / 16);
      constexpr int kAfterHalf = 16 + 1 + H + kV;  // loads issued after a tile's half 0
      static_assert(kAfterHalf < 64, "vmcnt range");
      unsigned char* ebase = smem_raw + (size_t)w * 2 * kHalfBytes;
      const T* erow0 = sc.E + ((size_t)b * n) * n * DE;  // graph b
      // the transfers of EHalf::fetch, written out: through that helper the
      // compiler allocates this loop's registers differently (3811 against
      // 3508 instructions, more accumulator-register copies)
      auto fetch_half = [&](int jt, int half, bool valid) {
        const int j = 16 * jt + 8 * half + (l >> 3);  // lane l: key j, 16-byte piece l % 8
        const int jc = j < n ? j : n - 1;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int ir = i0 + r < n ? i0 + r : n - 1;
          const T* src = valid ? erow0 + ((size_t)ir * n + jc) * DE + (l & 7) * 8 : zeros<T>() + (l & 15) * 8;
          __builtin_amdgcn_global_load_lds((const void*)src,
                                           (__attribute__((address_space(3))) void*)(ebase + half * kHalfBytes + r * kRowPitch),
                                           16, 0, kCpolStream);
        }
      };
      uint32_t mk_raw;
      bool k_in;
      auto key_mask_raw = [&](int jt) {  // raw byte; the select happens at the use
        const int j = 16 * jt + li;
        k_in = j < n;
        mk_raw = sc.mask_b[k_in ? j : n - 1];
      };
      auto film_half = [&](int half, const f32x4& fc, float (&R)[4][16]) {
#pragma unroll
        for (int k = 0; k < 8; ++k) sc.film(EHalf<T, DE>::frag(ebase + half * kHalfBytes, li, lg, k), fc, R, 8 * half + k);
      };
      if (sc.mi_any && w < JT) {  // uniform per wave
        Frag<T, DH / 4> kf[H];
        Frag<T, 4> vf[H][DH / 16];
        fetch_half(w, 0, true);
        fetch_half(w, 1, true);
        key_mask_raw(w);
        sc.load_k(w, kf);
        sc.load_v(w, vf);
        for (int jt = w; jt < JT; jt += kWaves) {
          const int jn = jt + kWaves;
          const bool more = jn < JT;  // uniform
          const f32x4 fc = sc.film_start();
          float R[4][16];
          __builtin_amdgcn_sched_barrier(0);
          wait_vmcnt<kAfterHalf>();  // half 0 of this tile in LDS
          __builtin_amdgcn_sched_barrier(0);
          film_half(0, fc, R);
          wait_lgkmcnt0();  // half 0 read: it may be refetched
          __builtin_amdgcn_sched_barrier(0);
          fetch_half(jn, 0, more);
          // half 1 of this tile, its mask byte, K and V: everything but the
          // next tile's half 0 just issued (loaded a tile ago, K and V are in
          // by now; waiting here keeps the compiler from waiting for the
          // whole prefetch at their uses)
          wait_vmcnt<16>();
          __builtin_amdgcn_sched_barrier(0);
          film_half(1, fc, R);
          wait_lgkmcnt0();
          __builtin_amdgcn_sched_barrier(0);
          fetch_half(jn, 1, more);
          const uint32_t bits = key_bits(k_in ? mk_raw : 0u);
          key_mask_raw(jn);
          __builtin_amdgcn_sched_barrier(0);
          f32x4 S[H];
          sc.qk(kf, S);
          sc.load_k(jn, kf);
          float u[H][4];
          sc.scores_from(R, S, bits, u);
          online_step(u, vf);
          sc.load_v(jn, vf);
        }
        // the last tile's prefetch (zeros or clamped reads) still lands in
        // this wave's half tiles, which the O partials reuse after the barrier
        wait_vmcnt<0>();
      }
    } else {
      for (int jt = w; jt < JT; jt += kWaves) {
        const uint32_t bits = key_bits(mk);
        if (bits == 0u || !sc.mi_any) {  // tile without real pairs: the running statistics do not change
          mk = sc.key_mask_byte(jt + kWaves);
          continue;
        }
        Frag<T, DH / 4> kf[H];
        sc.load_k(jt, kf);
        Frag<T, 4> vf[H][DH / 16];
        float u[H][4];
        if constexpr (sizeof(T) == 2) {
          sc.load_v(jt, vf);
          ETile<T, DE> et;
          et.load(sc.E, b, n, i, sc.mi, 16 * jt, lg, bits);
          mk = sc.key_mask_byte(jt + kWaves);  // next tile's mask, behind this tile's loads
          sc.logits(et, kf, bits, u);
        } else {
          // float32: V after the scores, so that it is not live next to them
          mk = sc.key_mask_byte(jt + kWaves);
          sc.logits_streamed(16 * jt, kf, bits, u);
          sc.load_v(jt, vf);
        }
        online_step(u, vf);
      }
    }
    // combine lane groups, then waves (the barrier below also ends every
    // wave's use of the E half tiles in LDS, which the O partials then reuse)
#pragma unroll
    for (int h = 0; h < H; ++h) {
      const float lsum = lg_sum(l_run[h]);
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
    reduce_store_O<T, H, DH>(a, os_s, oacc, b, i0, w, li, lg, (uint32_t)(__ballot(sc.mi) & 0xffffull));
  } else {
    float u[MAXT][H][4];
    uint32_t mk[MAXT], bits[MAXT];
    // Issue order: mask bytes, then every small load, then the E stream; no
    // load waits on another, so the E stream leaves at once.
    const uint32_t mq = sc.query_mask_byte();
#pragma unroll
    for (int tt = 0; tt < MAXT; ++tt) mk[tt] = sc.key_mask_byte(w + kWaves * tt);
    sc.load_weights(a);
    // K and V of the wave's tile are loaded here with one tile per wave;
    // with several, each tile's K is loaded with its E and its V right
    // before its A V product (bounded register use)
    Frag<T, DH / 4> kf[H];
    Frag<T, 4> vf[H][DH / 16];
    if constexpr (MAXT == 1) {
      sc.load_k(w, kf);
      if constexpr (MODE != kLogits) sc.load_v(w, vf);
    }
    Updater<T, H, DE> up;
    if constexpr (MODE == kFused) up.init(a, li, lg);
    if constexpr (MAXT == 1 && sizeof(T) == 2) {
      // one tile per wave: every in-bounds pair is read, so the loads need
      // no mask bytes (masked values are discarded by the selects)
      ETile<T, DE> et;
      et.template load_all<true>(sc.E, b, n, i, 16 * w, lg);
      __builtin_amdgcn_sched_barrier(0);  // nothing that waits on a load moves above the E stream
      sc.mi = mq != 0u;
      bits[0] = key_bits(mk[0]);
      sc.template logits<false>(et, kf, bits[0], u[0]);
      if constexpr (MODE != kLogits)
        attn_rest<T, H, DH, DE, 1, MODE, kKeepE>(a, sc, u, bits, vf, os_s, red_s, et, up);
    } else {
      sc.mi = mq != 0u;
#pragma unroll
      for (int tt = 0; tt < MAXT; ++tt) bits[tt] = key_bits(mk[tt]);
      if constexpr (MODE != kLogits) {
        if ((__ballot(sc.mi) & 0xffffull) == 0ull) {
          // no real query in the block (uniform): A, O and E' rows are all +0.0
          zero_block<T, H, DH, DE, MAXT, MODE == kFused>(a, b, i0, i, w, lg);
          return;
        }
      }
#pragma unroll
      for (int tt = 0; tt < MAXT; ++tt) {
        if constexpr (MAXT > 1) sc.load_k(w + kWaves * tt, kf);
        if constexpr (sizeof(T) == 2) {
          ETile<T, DE> et;
          et.load(sc.E, b, n, i, sc.mi, 16 * (w + kWaves * tt), lg, bits[tt]);
          sc.logits(et, kf, bits[tt], u[tt]);
        } else {
          sc.logits_streamed(16 * (w + kWaves * tt), kf, bits[tt], u[tt]);
        }
      }
      if constexpr (MODE != kLogits) {
        ETile<T, DE> unused;
        attn_rest<T, H, DH, DE, MAXT, MODE, false>(a, sc, u, bits, vf, os_s, red_s, unused, up);
      }
    }
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
    }
  }
}

// ------------------------------------------------------------------ fused layer, several key tiles per wave

// Where lanes of fused_stream_kernel whose pair lies outside the n x n layout
// store their edge outputs (a lane's de / 4 channels of one key; nothing
// reads it).
__device__ __align__(16) uint32_t kEdgeSink[8];

// Single-pass layer (scores, softmax, A, O and the residual edge update) for
// 64 < n <= 64 MAXT in bfloat16 with de = 64. One block per (graph, 16-query
// block); wave w owns key tiles w, w + kWaves, ... (MAXT of them) and reads
// only its live ones (some real key, in a block with a real query). The E
// tiles of a wave (MAXT x 32 KB) do not fit on chip next to the rest, so each
// live tile crosses from HBM twice, both times through LDS in half tiles
// with the next half tile in flight: for the scores, and after the softmax
// over the whole row for the update. The stream does not stop between the
// two phases: the last score step prefetches the first update tile.
// The global-to-LDS transfers are not tracked by the compiler's waits, so the
// kernel issues its memory operations in a fixed order and waits explicitly:
//   score step:  [half 0 of the next tile] [half 1 of the next tile]
//   update step: [half 0 of the next tile] [E' stores, keys 0-7]
//                [half 1 of the next tile] [E' stores, keys 8-15]
// Loads retire in issue order; the kernel does not rely on stores retiring
// in order with older loads (the compiler does not assume it either), so a
// wait counts only the loads issued after the one it waits for. K and V
// fragments load outside these loops; A, and the E' zeros of the tiles
// without a real key, are stored after the update loop.
template <typename T, int H, int DH, int DE, int MAXT>
__global__ __launch_bounds__(kThreads) void fused_stream_kernel(LayerArgs a) {
  static_assert(sizeof(T) == 2 && DE == 64 && MAXT >= 2, "bfloat16, de = 64, several key tiles");
  using EH = EHalf<T, DE>;
  using Up = Updater<T, H, DE>;
  constexpr int D = H * DH;
  constexpr int kEBytes = kWaves * 2 * EH::kBytes;
  static_assert(kWaves * 16 * kOPitch<D> * 4 <= kEBytes, "the O partials reuse the E half tiles");
  __shared__ __align__(16) unsigned char smem_raw[kEBytes];
  __shared__ float red_s[2][kWaves][H][16];
  const int tid = threadIdx.x, l = tid & 63, li = l & 15, lg = l >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: the wave's tiles and waits are scalar
  int ib, b;
  if (a.order) {  // the work order written by qkv_kernel (uniform)
    const int L = a.order[blockIdx.y * gridDim.x + blockIdx.x];
    ib = L % (int)gridDim.x;
    b = L / (int)gridDim.x;
  } else {
    xcd_block(ib, b);
  }
  const int i0 = ib * 16;
  Scorer<T, H, DH, DE> sc;
  sc.setup(a, b, i0);
  const int JT = sc.JT, n = a.n, i = sc.i;
  // mask bytes first: which tiles are live decides what the E stream reads
  const uint32_t mq = sc.query_mask_byte();
  uint32_t mk[MAXT];
#pragma unroll
  for (int tt = 0; tt < MAXT; ++tt) mk[tt] = sc.key_mask_byte(w + kWaves * tt);
  sc.load_weights(a);
  Up up;
  up.init(a, li, lg);
  sc.mi = mq != 0u;
  if ((__ballot(sc.mi) & 0xffffull) == 0ull) {  // no real query (uniform): zeros only
    zero_block<T, H, DH, DE, MAXT, true>(a, b, i0, i, w, lg);
    return;
  }
  // every small load has landed before the stream starts: afterwards the
  // loops below hold no older load the compiler would have to wait for
  wait_vmcnt<0>();
  uint32_t bits[MAXT];
  uint32_t live = 0u;  // bit tt: tile w + kWaves tt has a real key (uniform)
#pragma unroll
  for (int tt = 0; tt < MAXT; ++tt) {
    bits[tt] = key_bits(mk[tt]);  // 0 past the padded size
    if (bits[tt] != 0u) live |= 1u << tt;
  }
  const int first = live ? __builtin_ctz(live) : 0;
  unsigned char* ebase = smem_raw + (size_t)w * 2 * EH::kBytes;
  const T* Eb = sc.E + (size_t)b * n * n * DE;
  auto fetch = [&](int tt, int half) { EH::fetch(Eb, n, i0, w + kWaves * tt, half, ebase, l); };
  // the update's re-read is the tile's last use: streaming cache policy
  // (75.0 against 77.2 us at B = 32, n = 192)
  auto fetch_last = [&](int tt, int half) {
    EH::template fetch<kCpolStream>(Eb, n, i0, w + kWaves * tt, half, ebase, l);
  };
  // Both loops below walk the live tiles at run time. The score loop issues
  // the same transfers in every step (after the last score tile it fetches
  // the first update tile); the update loop fetches only while a next tile
  // exists.

  // ---- scores: live tiles in order, the next one streaming in
  float u[MAXT][H][4];
#pragma unroll
  for (int q = 0; q < MAXT; ++q) Scorer<T, H, DH, DE>::no_keys(u[q]);
  // K of every tile of the wave up front (no load into registers crosses a
  // step of the loop, so leaving it waits for nothing)
  Frag<T, DH / 4> kall[MAXT][H];
#pragma unroll
  for (int q = 0; q < MAXT; ++q) sc.load_k(w + kWaves * q, kall[q]);
  if (live) {  // uniform
    fetch(first, 0);
    fetch(first, 1);
  }
#pragma unroll 1
  for (uint32_t m = live; m != 0u; m &= m - 1u) {
    const int tt = __builtin_ctz(m);
    const uint32_t rest = m & (m - 1u);
    const int nt = rest ? __builtin_ctz(rest) : first;  // after the last score tile: the first update tile
    uint32_t bt = 0u;
    Frag<T, DH / 4> kf[H];
#pragma unroll
    for (int q = 0; q < MAXT; ++q)
      if (q == tt) {
        bt = bits[q];
#pragma unroll
        for (int h = 0; h < H; ++h) kf[h] = kall[q][h];
      }
    const f32x4 fc = sc.film_start();
    float R[4][16];
    Frag<T, DE / 4> ef[8];
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<16>();  // half 0 of this tile (newer: its half 1)
    EH::frags8(ebase, li, lg, ef);
    __builtin_amdgcn_sched_barrier(0);
    fetch(nt, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < 8; ++k) sc.film(ef[k], fc, R, k);
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<16>();  // half 1 of this tile (newer: the half 0 just issued)
    EH::frags8(ebase + EH::kBytes, li, lg, ef);
    __builtin_amdgcn_sched_barrier(0);
    fetch(nt, 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < 8; ++k) sc.film(ef[k], fc, R, 8 + k);
    f32x4 S[H];
    sc.qk(kf, S);
    float ut[H][4];
    sc.scores_from(R, S, bt, ut);
#pragma unroll
    for (int q = 0; q < MAXT; ++q)
      if (q == tt)
#pragma unroll
        for (int h = 0; h < H; ++h)
#pragma unroll
          for (int r = 0; r < 4; ++r) u[q][h][r] = ut[h][r];
  }

  // ---- softmax over the whole row (lane groups by register swaps, waves
  // through LDS); the V fragments of the wave's tiles load meanwhile (all of
  // them, unconditionally: tiles past the padded size read the last one)
  Frag<T, 4> vf[MAXT][H][DH / 16];
#pragma unroll
  for (int tt = 0; tt < MAXT; ++tt) sc.load_v(w + kWaves * tt, vf[tt]);
#pragma unroll
  for (int h = 0; h < H; ++h) {
    float m = kNegInf;
#pragma unroll
    for (int tt = 0; tt < MAXT; ++tt)
#pragma unroll
      for (int r = 0; r < 4; ++r) m = fmaxf(m, u[tt][h][r]);
    m = lg_max(m);
    if (lg == 0) red_s[0][w][h][li] = m;
  }
  lds_barrier();  // the update's first tile stays in flight
  float inv[H];
#pragma unroll
  for (int h = 0; h < H; ++h) {
    float M = kNegInf;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, red_s[0][ww][h][li]);
    // exp(u - M) as 2^(u log2 e - M log2 e); masked logits give exactly 0
    const float mb = (M == kNegInf) ? 0.f : M * kLog2e;
    float s = 0.f;
#pragma unroll
    for (int tt = 0; tt < MAXT; ++tt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(u[tt][h][r], kLog2e, -mb));
        u[tt][h][r] = p;
        s += p;
      }
    s = lg_sum(s);
    if (lg == 0) red_s[1][w][h][li] = s;
  }
  lds_barrier();
#pragma unroll
  for (int h = 0; h < H; ++h) {
    float L = 0.f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) L += red_s[1][ww][h][li];
    inv[h] = (L > 0.f) ? __builtin_amdgcn_rcpf(L) : 0.f;
  }

  // ---- A in bfloat16 (stored later), O^T += V^T A^T over the live tiles
  f32x4 oacc[H][DH / 16];
#pragma unroll
  for (int h = 0; h < H; ++h)
#pragma unroll
    for (int tc = 0; tc < DH / 16; ++tc) oacc[h][tc] = f32x4{0.f, 0.f, 0.f, 0.f};
  Frag<T, 4> ak[MAXT][H];
#pragma unroll
  for (int tt = 0; tt < MAXT; ++tt) {
#pragma unroll
    for (int h = 0; h < H; ++h) {
      float p[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) p[r] = u[tt][h][r] * inv[h];
      ak[tt][h].set(p);
    }
    if ((live >> tt) & 1u) {
#pragma unroll
      for (int h = 0; h < H; ++h)
#pragma unroll
        for (int tc = 0; tc < DH / 16; ++tc) oacc[h][tc] = mma(oacc[h][tc], vf[tt][h][tc], ak[tt][h]);
    }
  }

  // ---- residual edge update of the live tiles, E streamed through LDS again
  up.finish();
  T* Eout = static_cast<T*>(a.E_out);
  const bool iin = i < n;
  const size_t rowoff = ((size_t)b * n + (iin ? i : 0)) * n * DE + lg * (DE / 4);
  // every lane stores each key (pairs outside the n x n layout to the sink),
  // so that every half tile issues the same stores
  static_assert(DE / 4 * sizeof(T) <= sizeof(kEdgeSink), "sink size");
  T* sink = reinterpret_cast<T*>(kEdgeSink);
  wait_vmcnt<0>();  // the first update tile has landed (and every load before it)
#pragma unroll 1
  for (uint32_t m = live; m != 0u; m &= m - 1u) {
    const int tt = __builtin_ctz(m);
    const uint32_t rest = m & (m - 1u);
    const int nt = rest ? __builtin_ctz(rest) : tt;
    const int j0 = 16 * (w + kWaves * tt);
    Frag<T, 4> akc[H];
    uint32_t bt = 0u;
#pragma unroll
    for (int q = 0; q < MAXT; ++q)
      if (q == tt) {
        bt = bits[q];
#pragma unroll
        for (int h = 0; h < H; ++h) akc[h] = ak[q][h];
      }
    float R[4][Up::RW];
    up.head_operand(akc, R);
    const bool full = tile_full(sc.mi, bt);
    const uint32_t okj = sc.mi ? bt : 0u;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      __builtin_amdgcn_sched_barrier(0);
      // this half tile in LDS. Newer are the stores of the two half tiles
      // before it and the half tile fetched between them (if any); only the
      // newer loads are counted (for the first tile everything has landed
      // already)
      if (half == 0 || rest) wait_vmcnt<16>(); else wait_vmcnt<0>();
      Frag<T, DE / 4> ef[8];
      EH::frags8(ebase + half * EH::kBytes, li, lg, ef);
      __builtin_amdgcn_sched_barrier(0);
      if (rest) fetch_last(nt, half);  // uniform
      __builtin_amdgcn_sched_barrier(0);
      if (full) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int jj = 8 * half + k;
          up.template step_to<true>(ef[k], Eout + rowoff + (size_t)(j0 + jj) * DE, true, R, jj);
        }
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int jj = 8 * half + k;
          T* dst = (iin && j0 + jj < n) ? Eout + rowoff + (size_t)(j0 + jj) * DE : sink;
          up.template step_to<false>(ef[k], dst, (okj >> jj) & 1u, R, jj);
        }
      }
    }
  }
  // the last fetches land in LDS before the O partials reuse it (only
  // stores are newer: wait for everything)
  wait_vmcnt<0>();
  lds_barrier();
  const uint32_t qbits = (uint32_t)(__ballot(sc.mi) & 0xffffull);
  float* os_s = reinterpret_cast<float*>(smem_raw);
  o_partials_to_lds<H, DH>(os_s, oacc, w, li, lg);
  lds_barrier();
  o_reduce_store<T, H, DH>(a, os_s, b, i0, qbits);

  // ---- A of every tile of the wave, and the E' zeros of the dead tiles
  T* Ag = static_cast<T*>(a.A);
#pragma unroll
  for (int tt = 0; tt < MAXT; ++tt) {
    const int jt = w + kWaves * tt, j0 = 16 * jt, jb = j0 + 4 * lg;
    if (jt >= JT) continue;  // uniform
    if ((n & 3) == 0) {  // uniform: 4 keys in or out together, one vector store
      if (iin && jb < n) {
#pragma unroll
        for (int h = 0; h < H; ++h) ak[tt][h].store(Ag + (((size_t)b * H + h) * n + i) * n + jb);
      }
    } else if (iin) {
#pragma unroll
      for (int h = 0; h < H; ++h) {
        T* row = Ag + (((size_t)b * H + h) * n + i) * n;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (jb + r < n) Num<T>::st(row + jb + r, ak[tt][h].get(r));
      }
    }
    if (!((live >> tt) & 1u)) zero_edge_tile<T, DE>(Eout, b, n, i, j0, lg);
  }
}

// ------------------------------------------------------------------ update kernel

// Grid (NP/16 query blocks x ceil(NP/64) key groups, B), key group fastest:
// wave w of key group z takes key tile 4*z + w. Blocks running together then
// cover whole rows of E (contiguous memory) rather than one column stripe of
// many rows. kReadA reads A from the forward's output; kRecompute re-runs the
// score stage and takes A = exp(u - lse) from pass 1's statistics;
// kRecomputeU (unnormalized variant) re-runs it and takes the logit u itself.
// The E fragments of the tile are read once (bfloat16) and serve both stages.
// Two-pass pass 2 with an A buffer: this lane's four keys jb .. jb + 3 of
// query i, every head, into A [B, H, n, n] (the bfloat16 operand the update
// uses, 0 at masked pairs); keys or queries outside the n x n map are not
// written.
template <typename T, int H>
__device__ __forceinline__ void store_a_keys(T* Ag, int b, int n, int i, int jb, const Frag<T, 4> (&ak)[H]) {
  if ((n & 3) == 0) {  // uniform: 4 keys in or out together, one vector store
    if (i < n && jb < n) {
#pragma unroll
      for (int h = 0; h < H; ++h) ak[h].store(Ag + (((size_t)b * H + h) * n + i) * n + jb);
    }
  } else if (i < n) {
#pragma unroll
    for (int h = 0; h < H; ++h) {
      T* row = Ag + (((size_t)b * H + h) * n + i) * n;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (jb + r < n) Num<T>::st(row + jb + r, ak[h].get(r));
    }
  }
}

template <typename T, int H, int DH, int DE, int MODE>
__global__ __launch_bounds__(kThreads) void update_kernel(LayerArgs a) {
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, li = l & 15, lg = l >> 4;
  const int KG = (a.NP + kWaves * 16 - 1) / (kWaves * 16);  // key groups
  const int b = blockIdx.y, i0 = (blockIdx.x / KG) * 16, i = i0 + li;
  const int n = a.n, NP = a.NP, JT = NP / 16;
  const int jt = (blockIdx.x % KG) * kWaves + w, j0 = 16 * jt;
  constexpr bool kKeepE = sizeof(T) == 2;
  Scorer<T, H, DH, DE> sc;
  sc.setup(a, b, i0);
  // Issue order: mask bytes and every small load (none conditional), then
  // the tile test, then the E stream.
  const uint32_t mq = sc.query_mask_byte();
  const uint32_t mk = sc.key_mask_byte(jt);
  Updater<T, H, DE> up;
  // recompute modes: the update weights and the row statistics are loaded
  // after the score stage (not live next to the E tile and the FiLM rows)
  constexpr bool kRe = MODE == kRecompute || MODE == kRecomputeU;
  if constexpr (!kRe) up.init(a, li, lg);
  float A[H][4];
  Frag<T, DH / 4> kf[H];
  if constexpr (kRe) {
    sc.load_weights(a);
    sc.load_k(jt, kf);
  } else {
    // entries outside the n x n map read entry (0, 0) of the head and are zeroed
    const T* Ag = static_cast<const T*>(a.A);
    const int jb = j0 + 4 * lg;
    if ((n & 3) == 0) {  // uniform: 4 consecutive keys in or out together
      const bool ok = jt < JT && i < n && jb < n;
      Frag<T, 4> f[H];
#pragma unroll
      for (int h = 0; h < H; ++h) f[h].load(Ag + ((size_t)b * H + h) * n * n + (ok ? (size_t)i * n + jb : 0));
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int h = 0; h < H; ++h)
#pragma unroll
        for (int r = 0; r < 4; ++r) A[h][r] = ok ? f[h].get(r) : 0.f;
    } else {
      T raw[H][4];
#pragma unroll
      for (int h = 0; h < H; ++h)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bool ok = jt < JT && i < n && jb + r < n;
          raw[h][r] = Ag[((size_t)b * H + h) * n * n + (ok ? (size_t)i * n + jb + r : 0)];
        }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int h = 0; h < H; ++h)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bool ok = jt < JT && i < n && jb + r < n;
          A[h][r] = ok ? Num<T>::ld(&raw[h][r]) : 0.f;
        }
    }
  }
  sc.mi = mq != 0u;
  const uint32_t bits = key_bits(mk);
  if ((__ballot(sc.mi) & 0xffffull) == 0ull || bits == 0u) {  // no real pair in the tile (uniform): zeros only
    if (jt < JT) zero_edge_tile<T, DE>(static_cast<T*>(a.E_out), b, n, i, j0, lg);
    if constexpr (MODE == kRecompute) {
      if (a.A != nullptr && jt < JT) {  // uniform: the map is asked for
        Frag<T, 4> z[H];
#pragma unroll
        for (int h = 0; h < H; ++h) z[h].zero();
        store_a_keys<T, H>(static_cast<T*>(a.A), b, n, i, j0 + 4 * lg, z);
      }
    }
    return;
  }
  ETile<T, DE> et;
  if constexpr (kKeepE) et.load(sc.E, b, n, i, sc.mi, j0, lg, bits);
  if constexpr (kRe) {
    float u[H][4];
    if constexpr (kKeepE) {
      // S first, so that K and Q are dead while the E tile and the FiLM rows
      // are live (fewer registers live at once; the E tile alone takes 128)
      f32x4 S[H];
      sc.qk(kf, S);
      __builtin_amdgcn_sched_barrier(0);
      const f32x4 fc = sc.film_start();
      float R[4][16];
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) sc.film(et.f[jj], fc, R, jj);
      sc.scores_from(R, S, bits, u);
    } else {
      sc.logits_streamed(j0, kf, bits, u);
    }
    up.init(a, li, lg);
    if constexpr (MODE == kRecomputeU) {
      // unnormalized variant: the operand is the logit itself, 0 at masked pairs
#pragma unroll
      for (int h = 0; h < H; ++h)
#pragma unroll
        for (int r = 0; r < 4; ++r) A[h][r] = u[h][r] == kNegInf ? 0.f : u[h][r];
    } else {
      float L[H];
#pragma unroll
      for (int h = 0; h < H; ++h) L[h] = a.lse[((size_t)b * H + h) * NP + i];
#pragma unroll
      for (int h = 0; h < H; ++h)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          A[h][r] = (u[h][r] == kNegInf || L[h] == kNegInf) ? 0.f : __expf(u[h][r] - L[h]);
    }
  }
  up.finish();
  const bool full = tile_full(sc.mi, bits);
  Frag<T, 4> ak[H];
#pragma unroll
  for (int h = 0; h < H; ++h) ak[h].set(A[h]);
  if constexpr (MODE == kRecompute) {
    if (a.A != nullptr && jt < JT) store_a_keys<T, H>(static_cast<T*>(a.A), b, n, i, j0 + 4 * lg, ak);
  }
  if (jt < JT)
    up.template tile<kKeepE>(et, sc.E, static_cast<T*>(a.E_out), b, n, i, sc.mi, j0, lg, bits, full, ak, [] {});
}

// One wave's E tile (16 queries x 16 keys x DE, bfloat16) into LDS with
// global-to-LDS loads of 16 bytes per lane: piece q of key jj of lane l lands
// at dst[(jj * DE / 32 + q) * 64 + l], the lane order of the register
// fragments. Pairs outside the n x n layout read the nearest one inside it.
// (The source goes to the builtin as const void*: another pointer type makes
// the host pass drop the kernel's launch stub without an error.)
template <typename T, int DE>
__device__ __forceinline__ void e_tile_to_lds(const T* E, int b, int n, int i, int j0, int lg, u32x4* dst) {
  constexpr int LPK = DE / 32;
  const T* row = E + ((size_t)b * n + (i < n ? i : n - 1)) * n * DE + lg * (DE / 4);
#pragma unroll
  for (int jj = 0; jj < 16; ++jj) {
    const int j = j0 + jj;
    const T* src = row + (size_t)(j < n ? j : n - 1) * DE;
#pragma unroll
    for (int q = 0; q < LPK; ++q)
      __builtin_amdgcn_global_load_lds((const void*)(src + 8 * q),
                                       (__attribute__((address_space(3))) void*)(dst + (jj * LPK + q) * 64), 16, 0, 0);
  }
}

// Two-pass pass 2 (and the unnormalized update) in bfloat16, as a persistent
// pipeline. Work items are (graph, 16-query block, group of 4 key tiles), key
// group fastest, so the blocks running at one time cover whole rows of E.
// Every block walks items blockIdx.x, blockIdx.x + gridDim.x, ...; wave w of
// an item owns key tile 4 * group + w. While a wave computes one item from
// registers, its next item's E tile streams into the wave's own LDS region
// through global-to-LDS loads (16 bytes per lane, in the lane order of the
// register fragments), so the E reads of the next item overlap the score
// stage, the update and the E' stores of this one. The global-to-LDS loads
// are not tracked by the compiler's waits: the kernel waits explicitly (all
// vector memory operations before reading the tile, and its own LDS reads
// before the next tile may overwrite it).
// Every pair of a tile is read (masked values are discarded by the selects).
template <typename T, int H, int DH, int DE, int MODE>
__global__ __launch_bounds__(kThreads) void update_pipe_kernel(LayerArgs a, int items) {
  static_assert(sizeof(T) == 2 && DE % 32 == 0, "bfloat16, 16-byte pieces");
  constexpr int LPK = DE / 32;   // 16-byte pieces per lane and key
  constexpr int NL = 16 * LPK;   // per tile
  __shared__ u32x4 ebuf[kWaves][NL][64];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, li = l & 15, lg = l >> 4;
  const int n = a.n, NP = a.NP, JT = NP / 16, QB = NP / 16, KG = (JT + kWaves - 1) / kWaves;
  const int G = gridDim.x;
  int it = blockIdx.x;
  if (it >= items) return;  // uniform
  struct Item {
    int b, i0, jt;
  };
  auto decode = [&](int x) {
    Item r;
    const int rest = x / KG;
    r.jt = (x - rest * KG) * kWaves + w;
    r.i0 = (rest % QB) * 16;
    r.b = rest / QB;
    return r;
  };
  Scorer<T, H, DH, DE> sc;
  Frag<T, DH / 4> kf[H];
  float L[H];
  // raw mask bytes and whether their node exists: the select happens at the
  // use (the next iteration), so nothing waits on these loads early
  uint32_t mq, mk;
  bool q_in, k_in;
  auto issue_small = [&](const Item& m) {
    sc.setup(a, m.b, m.i0);
    const int i = m.i0 + li, j = 16 * m.jt + li;
    q_in = i < n;
    k_in = j < n;
    mq = sc.mask_b[q_in ? i : n - 1];
    mk = sc.mask_b[k_in ? j : n - 1];
    sc.load_queries(a);
    sc.load_k(m.jt, kf);
    if constexpr (MODE == kRecompute) {
#pragma unroll
      for (int h = 0; h < H; ++h) L[h] = a.lse[((size_t)m.b * H + h) * NP + sc.i];
    }
  };
  const T* Eg = static_cast<const T*>(a.E);
  Item cur = decode(it);
  e_tile_to_lds<T, DE>(Eg, cur.b, n, cur.i0 + li, 16 * cur.jt, lg, &ebuf[w][0][0]);
  issue_small(cur);  // sets the scorer's lane indices, which load_film uses
  sc.load_film(a);
  Updater<T, H, DE> up;
  up.init(a, li, lg);
  up.finish();
  for (;;) {
    const int nx = it + G;
    const bool more = nx < items;  // uniform
    __builtin_amdgcn_sched_barrier(0);
    // this item's E tile and small loads have landed (newer are only the
    // previous item's E' stores, which are not counted on to retire in order
    // with older loads: wait for everything)
    wait_vmcnt<0>();
    __builtin_amdgcn_sched_barrier(0);
    ETile<T, DE> et;
#pragma unroll
    for (int jj = 0; jj < 16; ++jj)
#pragma unroll
      for (int q = 0; q < LPK; ++q) {
        const u32x4 v = ebuf[w][jj * LPK + q][l];
        et.f[jj].w[4 * q] = v.x; et.f[jj].w[4 * q + 1] = v.y; et.f[jj].w[4 * q + 2] = v.z; et.f[jj].w[4 * q + 3] = v.w;
      }
    wait_lgkmcnt0();
    __builtin_amdgcn_sched_barrier(0);
    const Item nxt = decode(more ? nx : it);
    if (more) e_tile_to_lds<T, DE>(Eg, nxt.b, n, nxt.i0 + li, 16 * nxt.jt, lg, &ebuf[w][0][0]);
    __builtin_amdgcn_sched_barrier(0);  // the tile's loads are issued before this item's work
    // this item: logits, A, then the next item's small loads, then the update
    const int i = cur.i0 + li, j0 = 16 * cur.jt;
    const bool mi = q_in && mq != 0u;
    const uint32_t bits = key_bits(k_in ? mk : 0u);
    const bool live = (__ballot(mi) & 0xffffull) != 0ull && bits != 0u && cur.jt < JT;  // uniform
    sc.mi = mi;
    float A[H][4];
    {
      f32x4 S[H];
      sc.qk(kf, S);
      const f32x4 fc = sc.film_start();
      float R[4][16];
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) sc.film(et.f[jj], fc, R, jj);
      float u[H][4];
      sc.scores_from(R, S, bits, u);
#pragma unroll
      for (int h = 0; h < H; ++h)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if constexpr (MODE == kRecomputeU)
            A[h][r] = u[h][r] == kNegInf ? 0.f : u[h][r];
          else
            A[h][r] = (u[h][r] == kNegInf || L[h] == kNegInf) ? 0.f : __expf(u[h][r] - L[h]);
        }
    }
    const bool full = tile_full(mi, bits);
    const int b = cur.b, jt = cur.jt;
    if (more) issue_small(nxt);
    if constexpr (MODE == kRecompute) {
      if (a.A != nullptr && jt < JT) {  // uniform: the map is asked for (0 at masked pairs)
        Frag<T, 4> aq[H];
#pragma unroll
        for (int h = 0; h < H; ++h) aq[h].set(A[h]);
        store_a_keys<T, H>(static_cast<T*>(a.A), b, n, i, j0 + 4 * lg, aq);
      }
    }
    if (live) {
      Frag<T, 4> ak[H];
#pragma unroll
      for (int h = 0; h < H; ++h) ak[h].set(A[h]);
      up.template tile<true>(et, sc.E, static_cast<T*>(a.E_out), b, n, i, mi, j0, lg, bits, full, ak, [] {});
    } else if (jt < JT) {
      zero_edge_tile<T, DE>(static_cast<T*>(a.E_out), b, n, i, j0, lg);
    }
    if (!more) break;
    it = nx;
    cur = nxt;
  }
}

// ------------------------------------------------------------------ backward

// Gradients of one layer (forward and residual edge update), single-pass
// shapes (the stored A is reused), from the loss gradients dO of
// the node output and dE' of the edge output. Per real pair (i, j), head h:
//   dA = dO_i . V_j + sum_c W_e[c, h] dE'_ij[c]        (through A V and E')
//   D_i = sum_j A_ij dA_ij,  du = A (dA - D)             (softmax)
//   ds = du gamma_y gamma_e,  dgamma_e = du gamma_y s,  dbeta_e = du gamma_y
//   (u = (s gamma_e + beta_e) gamma_y + beta_y, s = q_i . k_j / sqrt(dh))
//   dE_ij = dE'_ij + W_em^T dgamma_e + W_ea^T dbeta_e   (0 at masked pairs)
//   dQ = r ds K, dK = r ds^T Q, dV = A^T dO per (graph, head); the weight
//   gradients are sums over real pairs (edge FiLM, W_e) or real rows (Q, K,
//   V projections) or graphs (global FiLM).
// A is the forward's stored map (bfloat16 in bf16 mode): the backward of a
// rounding point counts as the identity.

// Four consecutive values of type T (8 or 16 bytes) from floats.
template <typename T>
__device__ __forceinline__ void store4(T* p, const float* v) {
  if constexpr (sizeof(T) == 2) {
    *reinterpret_cast<u32x2*>(p) = u32x2{pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3])};
  } else {
    *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
  }
}

// bwd_prep: V in row layout [B, H, NP, dh] (the forward keeps V^T), one
// (graph, head, 64 keys) tile per block through LDS, 16-byte reads and
// writes on both sides.
template <typename T, int H, int DH, int DE>
__global__ __launch_bounds__(kThreads) void bwd_prep_kernel(LayerArgs a, BwdArgs g) {
  const int NP = a.NP;
  constexpr int EPC = 16 / (int)sizeof(T);
  const int JB = (NP + 63) / 64;
  __shared__ T vt_s[DH][64 + EPC];
  const int bh = blockIdx.x / JB, j0 = (blockIdx.x % JB) * 64;
  const T* src = static_cast<const T*>(a.Vt) + (size_t)bh * DH * NP;
  // NP is a multiple of 16: a chunk of EPC keys is wholly inside or outside
  for (int c = threadIdx.x; c < DH * 64 / EPC; c += kThreads) {
    const int t = c / (64 / EPC), jj = (c % (64 / EPC)) * EPC;
    if (j0 + jj < NP)
      *reinterpret_cast<u32x4*>(&vt_s[t][jj]) = *reinterpret_cast<const u32x4*>(src + (size_t)t * NP + j0 + jj);
  }
  __syncthreads();
  T* dst = static_cast<T*>(g.Vr) + (size_t)bh * NP * DH;
  for (int c = threadIdx.x; c < 64 * DH / EPC; c += kThreads) {
    const int jj = c / (DH / EPC), t0 = (c % (DH / EPC)) * EPC;
    if (j0 + jj < NP) {
      __align__(16) T v[EPC];
#pragma unroll
      for (int e = 0; e < EPC; ++e) v[e] = vt_s[t0 + e][jj];
      *reinterpret_cast<u32x4*>(dst + (size_t)(j0 + jj) * DH + t0) = *reinterpret_cast<const u32x4*>(v);
    }
  }
}

// bwd_pair: one block per (16 queries, graph, 16 WV keys), wave w = key tile
// WV blockIdx.z + w (WV = 4 waves, 64 keys, except kPairUse, which runs
// kWaves / kUseSplit). The row sums D_i = sum_j A_ij dA_ij span every key:
//   kPairAll  (n <= 64, one key block): D from the block's four waves;
//   kPairPart (64 < n): only dA, and the block's part of D into DP;
//   kPairUse  (64 < n): D as the sum of the key blocks' parts, then the rest;
//   kPairPartA (two-pass contexts, where A is not stored): as kPairPart, with
//     A recomputed from the logits and the forward's row statistics,
//     A = exp(u - lse_i) rounded to T (the operand the forward's update used),
//     and written to g.A for the kernels that follow.
enum PairMode : int { kPairAll = 0, kPairPart = 1, kPairUse = 2, kPairPartA = 3 };
template <typename T, int H, int DH, int DE, int PM, int WV = kWaves>
__global__ __launch_bounds__(WV * 64) void bwd_pair_kernel(LayerArgs a, BwdArgs g) {
  constexpr int D = H * DH, NCH = DE / 16;
  // Modes that write dE keep the dE' tile of step (1) in LDS for step (5)
  // (each lane reads back its own words), so dE' crosses HBM once
  constexpr bool kKeepDep = PM == kPairAll || PM == kPairUse;
  constexpr int NDW = Frag<T, DE / 4>::ND;  // words of one lane's fragment
  constexpr int NDC = NDW % 4 == 0 ? 4 : NDW;  // words per LDS access
  static_assert(WV == kWaves || PM == kPairUse, "the row sums of D over a block's waves need all four key tiles");
  __shared__ float red_s[WV][H][16];
  __shared__ float sum_s[WV][4 * H];
  __shared__ __align__(16) uint32_t dep_s[kKeepDep ? WV * 16 * NDW * 64 : 1];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, li = l & 15, lg = l >> 4;
  const int b = blockIdx.y, i0 = blockIdx.x * 16;
  // word group c of key jj of this lane: 16-byte pieces of consecutive lanes side by side
  auto dep_at = [&](int jj, int c) { return dep_s + (((w * 16 + jj) * (NDW / NDC) + c) * 64 + l) * NDC; };
  Scorer<T, H, DH, DE> sc;
  sc.setup(a, b, i0);
  const int n = a.n, NP = a.NP, JT = sc.JT, i = sc.i, jt = WV * blockIdx.z + w, j0 = 16 * jt;
  const int KB = (NP + 63) / 64;  // 64-key blocks of the row (the parts of D)
  const int KBZ = gridDim.z;      // key blocks of this launch (the slots of PS)
  const bool tile_ok = jt < JT;  // uniform per wave; waves past JT compute zeros
  const uint32_t mq = sc.query_mask_byte();
  const uint32_t mk = sc.key_mask_byte(jt);
  // kPairUse with at most kMaxKB key blocks: the key blocks' parts of D for
  // this lane group's heads are requested before any other load and summed
  // once the dE' tile is in flight, so their round trip hides under the
  // tile's instead of following the softmax backward's barrier
  constexpr int HPG = (H + 3) / 4, kMaxKB = 16;
  constexpr bool kUse = PM == kPairUse;
  __shared__ float d_s[kUse ? WV : 1][kUse ? H : 1][16];
  float dpx[kUse ? HPG : 1][kUse ? kMaxKB : 1];
  if constexpr (kUse) {
#pragma unroll
    for (int hh = 0; hh < HPG; ++hh) {
      const int h = lg * HPG + hh < H ? lg * HPG + hh : H - 1;
      const float* row = g.DP + (((size_t)b * H + h) * NP + i) * KB;
#pragma unroll
      for (int q = 0; q < kMaxKB; ++q) dpx[hh][q] = row[q < KB ? q : KB - 1];
    }
  }
  // kPairPartA: the forward's row statistics of this lane's query, requested
  // with the other small loads rather than where A is recomputed
  float Lr[PM == kPairPartA ? H : 1];
  if constexpr (PM == kPairPartA) {
#pragma unroll
    for (int h = 0; h < H; ++h) Lr[h] = a.lse[((size_t)b * H + h) * NP + i];
  }
  sc.load_weights(a);
  Frag<T, DH / 4> kf[H], vr[H], dof[H];
  sc.load_k(jt, kf);
  const int jc = tile_ok ? jt : JT - 1;
  const T* Vr = static_cast<const T*>(g.Vr);
  const T* dO = static_cast<const T*>(g.dO);
#pragma unroll
  for (int h = 0; h < H; ++h) {
    vr[h].load(Vr + (((size_t)b * H + h) * NP + 16 * jc + li) * DH + lg * (DH / 4));
    dof[h].load(i < n ? dO + ((size_t)b * n + i) * D + h * DH + lg * (DH / 4) : zeros<T>());
  }
  // A of this lane's query and keys j0 + 4 lg + r (0 outside the n x n map)
  float Av[H][4];
  if constexpr (PM != kPairPartA) {
    const T* Ag = static_cast<const T*>(g.A);
    const int jb = j0 + 4 * lg;
    if (n % 4 == 0) {  // uniform: the lane's four keys in one load
      const bool ok = i < n && jb < n;
#pragma unroll
      for (int h = 0; h < H; ++h) {
        Frag<T, 4> f;
        f.load(Ag + ((size_t)b * H + h) * n * n + (ok ? (size_t)i * n + jb : 0));
#pragma unroll
        for (int r = 0; r < 4; ++r) Av[h][r] = ok ? f.get(r) : 0.f;
      }
    } else {
#pragma unroll
      for (int h = 0; h < H; ++h)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = jb + r;
          const bool ok = i < n && j < n;
          const float v = Num<T>::ld(Ag + ((size_t)b * H + h) * n * n + (ok ? (size_t)i * n + j : 0));
          Av[h][r] = ok ? v : 0.f;
        }
    }
  }
  // W_e^T row li (head li) over this lane group's channels, for dA through E'
  Frag<T, DE / 4> wet;
  {
    const T* We = static_cast<const T*>(a.w_e);
    float v[DE / 4];
#pragma unroll
    for (int k = 0; k < DE / 4; ++k) {
      const int c = lg * (DE / 4) + k;
      const float x = Num<T>::ld(li < H ? We + (size_t)c * H + li : zeros<T>());
      v[k] = li < H ? x : 0.f;
    }
    wet.set(v);
  }
  // W_F^T rows for dE (operand A): row li of chunk ch is channel
  // (li/4)(DE/4) + 4 ch + li%4; slot s of lane group lg is FiLM row 4 lg + s
  // (rows 0..H-1: W_em, H..2H-1: W_ea, the rest zero)
  Frag<T, 4> wF[NCH];
  {
    const T* Wm = static_cast<const T*>(a.w_emul);
    const T* Wa = static_cast<const T*>(a.w_eadd);
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
      const int c = (li >> 2) * (DE / 4) + 4 * ch + (li & 3);
      float v[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int fr = 4 * lg + s;
        const T* p = fr < H ? Wm + (size_t)fr * DE + c : fr < 2 * H ? Wa + (size_t)(fr - H) * DE + c : zeros<T>();
        const float x = Num<T>::ld(p);
        v[s] = fr < 2 * H ? x : 0.f;
      }
      wF[ch].set(v);
    }
  }
  sc.mi = mq != 0u;
  const uint32_t bits = tile_ok ? key_bits(mk) : 0u;
  const uint32_t okb = (bits >> (4 * lg)) & (sc.mi ? 0xfu : 0u);  // real pairs of this lane's 4 keys
  const T* dEp = static_cast<const T*>(g.dEp);

  // (1) dA through E': W_e^T dE' per pair, from the dE' tile
  float dAe[H][4];
  {
    ETile<T, DE> dt;
    dt.load_all(dEp, b, n, i, j0, lg);
    if constexpr (kUse) {
      if (KB <= kMaxKB) {  // uniform; the parts in key-block order
#pragma unroll
        for (int hh = 0; hh < HPG; ++hh) {
          float x = 0.f;
#pragma unroll
          for (int q = 0; q < kMaxKB; ++q)
            if (q < KB) x += dpx[hh][q];
          if (lg * HPG + hh < H) d_s[w][lg * HPG + hh][li] = x;
        }
      }
    }
    if constexpr (kKeepDep) {
#pragma unroll
      for (int jj = 0; jj < 16; ++jj)
#pragma unroll
        for (int c = 0; c < NDW / NDC; ++c) {
          uint32_t* q = dep_at(jj, c);
          if constexpr (NDC == 4)
            *reinterpret_cast<u32x4*>(q) = u32x4{dt.f[jj].w[4 * c], dt.f[jj].w[4 * c + 1], dt.f[jj].w[4 * c + 2],
                                                 dt.f[jj].w[4 * c + 3]};
          else
#pragma unroll
            for (int k = 0; k < NDC; ++k) q[k] = dt.f[jj].w[NDC * c + k];
        }
    }
    float R2[4][16];
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) {
      const f32x4 F = mma(f32x4{0.f, 0.f, 0.f, 0.f}, wet, dt.f[jj]);
#pragma unroll
      for (int r = 0; r < 4; ++r) R2[jj >> 2][4 * (jj & 3) + r] = F[r];
    }
    lane_group_transpose<16>(R2);
#pragma unroll
    for (int h = 0; h < H; ++h)
#pragma unroll
      for (int r = 0; r < 4; ++r) dAe[h][r] = R2[h >> 2][4 * r + (h & 3)];
  }
  // (2) the FiLM rows (gamma_e, beta_e) from the E tile (not needed for D alone)
  float R[4][16];
  if constexpr (PM != kPairPart) {
    ETile<T, DE> et;
    et.load_all(sc.E, b, n, i, j0, lg);
    const f32x4 fc = sc.film_start();
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) sc.film(et.f[jj], fc, R, jj);
    lane_group_transpose<16>(R);
  }
  // (3) scores and dO . V (both as S^T = K Q^T: lane (li, lg) holds query li, keys 4 lg + r)
  f32x4 S[H], P[H];
  if constexpr (PM != kPairPart) sc.qk(kf, S);
#pragma unroll
  for (int h = 0; h < H; ++h) P[h] = mma(f32x4{0.f, 0.f, 0.f, 0.f}, vr[h], dof[h]);
  if constexpr (PM == kPairPartA) {
    // A = exp(u - lse_i) on real pairs, rounded to T, stored for what follows
    T* Aw = static_cast<T*>(const_cast<void*>(g.A));
#pragma unroll
    for (int h = 0; h < H; ++h) {
      const float L = Lr[h];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float gam = R[h >> 2][4 * r + (h & 3)];
        const float bet = R[(H + h) >> 2][4 * r + ((H + h) & 3)];
        const float u = ((S[h][r] * sc.scale) * gam + bet) * sc.gy[h] + sc.gy[H + h];
        const bool ok = ((okb >> r) & 1u) && L != kNegInf;
        Av[h][r] = ok ? Num<T>::rnd(__expf(u - L)) : 0.f;
      }
      // the lane's four keys in one store where rows of n keep them aligned
      const int jb = j0 + 4 * lg;
      T* dst = Aw + (((size_t)b * H + h) * n + i) * n + jb;
      if (n % 4 == 0) {  // uniform
        if (i < n && jb < n) store4<T>(dst, Av[h]);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (i < n && jb + r < n) Num<T>::st(dst + r, Av[h][r]);
      }
    }
  }
  // (4) the softmax backward per pair and head
  float dA[H][4];
#pragma unroll
  for (int h = 0; h < H; ++h) {
    float part = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      dA[h][r] = ((okb >> r) & 1u) ? P[h][r] + dAe[h][r] : 0.f;
      part += Av[h][r] * dA[h][r];
    }
    part = lg_sum(part);
    if (lg == 0) red_s[w][h][li] = part;
  }
  __syncthreads();
  if constexpr (PM == kPairPart || PM == kPairPartA) {
    // this key block's part of D for the 16 queries
    if (tid < H * 16) {
      const int h = tid >> 4, q = tid & 15, iq = i - li + q;
      float x = 0.f;
#pragma unroll
      for (int ww = 0; ww < WV; ++ww) x += red_s[ww][h][q];
      g.DP[(((size_t)b * H + h) * NP + iq) * KB + blockIdx.z] = x;
    }
    return;
  }
  float ds[H][4], dge[H][4], dbe[H][4];
  float sgy[H], sby[H], sge[H], sbe[H];
  // D_i per head: the sum of the key blocks' parts in key-block order. The
  // parts of four key blocks of every head are requested together (clamped
  // indices, the surplus discarded by a uniform condition), so a row of KB
  // parts costs ceil(KB / 4) round trips instead of H KB dependent ones.
  float Dv[H];
#pragma unroll
  for (int h = 0; h < H; ++h) Dv[h] = 0.f;
  if constexpr (PM == kPairAll) {
#pragma unroll
    for (int h = 0; h < H; ++h)
#pragma unroll
      for (int ww = 0; ww < WV; ++ww) Dv[h] += red_s[ww][h][li];
  } else if (kUse && KB <= kMaxKB) {  // summed after the tile loads (above)
    if constexpr (kUse) {
#pragma unroll
      for (int h = 0; h < H; ++h) Dv[h] = d_s[w][h][li];
    }
  } else {
    const float* dp = g.DP + ((size_t)b * H * NP + i) * KB;  // head h at + h NP KB
    for (int kb0 = 0; kb0 < KB; kb0 += 4) {
      float x[H][4];
#pragma unroll
      for (int h = 0; h < H; ++h)
#pragma unroll
        for (int q = 0; q < 4; ++q) x[h][q] = dp[(size_t)h * NP * KB + (kb0 + q < KB ? kb0 + q : KB - 1)];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (kb0 + q < KB)
#pragma unroll
          for (int h = 0; h < H; ++h) Dv[h] += x[h][q];
    }
  }
#pragma unroll
  for (int h = 0; h < H; ++h) {
    const float Dh = Dv[h];
    const float gyh = sc.gy[h];
    sgy[h] = sby[h] = sge[h] = sbe[h] = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool ok = (okb >> r) & 1u;
      const float du = ok ? Av[h][r] * (dA[h][r] - Dh) : 0.f;
      const float s = S[h][r] * sc.scale;
      const float gam = R[h >> 2][4 * r + (h & 3)];
      const float bet = R[(H + h) >> 2][4 * r + ((H + h) & 3)];
      ds[h][r] = ok ? du * gyh * gam : 0.f;
      dge[h][r] = ok ? du * gyh * s : 0.f;
      dbe[h][r] = du * gyh;
      sgy[h] += ok ? du * (s * gam + bet) : 0.f;
      sby[h] += du;
      sge[h] += dge[h][r];
      sbe[h] += dbe[h][r];
    }
  }
  const size_t dErow = ((size_t)b * n + (i < n ? i : 0)) * n * DE + lg * (DE / 4);
  // ds and dgamma_e / dbeta_e for the (graph, head) and pair-reduction kernels
  if (tile_ok) {
#pragma unroll
    for (int h = 0; h < H; ++h) {
      store4<float>(g.DS + (((size_t)b * H + h) * NP + i) * NP + j0 + 4 * lg, ds[h]);
      store4<T>(static_cast<T*>(g.DF) + (((size_t)b * 2 * H + h) * NP + i) * NP + j0 + 4 * lg, dge[h]);
      store4<T>(static_cast<T*>(g.DF) + (((size_t)b * 2 * H + H + h) * NP + i) * NP + j0 + 4 * lg, dbe[h]);
    }
  }
  // (5) dE = dE' + W_F^T dF per key: dF regrouped so that lane group lg holds
  // FiLM rows 4 lg .. 4 lg + 3 of every key (the FiLM output layout)
  float dFa[4][16];
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int rp = 0; rp < 4; ++rp)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int fr = 4 * x + r;
        dFa[x][4 * rp + r] = fr < H ? dge[fr < H ? fr : 0][rp] : fr < 2 * H ? dbe[fr >= H && fr < 2 * H ? fr - H : 0][rp] : 0.f;
      }
  lane_group_transpose<16>(dFa);
  if (tile_ok) {
    T* dE = static_cast<T*>(g.dE);
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) {
      const int j = j0 + jj;
      const bool inb = i < n && j < n;
      const bool real = sc.mi && ((bits >> jj) & 1u);
      Frag<T, 4> bq;
      bq.set(&dFa[jj >> 2][4 * (jj & 3)]);
      Frag<T, DE / 4> ef;
#pragma unroll
      for (int c = 0; c < NDW / NDC; ++c) {
        const uint32_t* q = dep_at(jj, c);
        if constexpr (NDC == 4) {
          const u32x4 v = *reinterpret_cast<const u32x4*>(q);
          ef.w[4 * c] = v.x; ef.w[4 * c + 1] = v.y; ef.w[4 * c + 2] = v.z; ef.w[4 * c + 3] = v.w;
        } else {
#pragma unroll
          for (int k = 0; k < NDC; ++k) ef.w[NDC * c + k] = q[k];
        }
      }
      float out[DE / 4];
#pragma unroll
      for (int ch = 0; ch < NCH; ++ch) {
        const f32x4 c = mma(f32x4{0.f, 0.f, 0.f, 0.f}, wF[ch], bq);
#pragma unroll
        for (int r = 0; r < 4; ++r) out[4 * ch + r] = real ? c[r] + ef.get(4 * ch + r) : 0.f;
      }
      if (inb) {
        Frag<T, DE / 4> of;
        of.set(out);
        of.store(dE + dErow + (size_t)j * DE);
      }
    }
  }
  // (6) sums over the block's pairs: dgamma_y, dbeta_y (per graph), b_emul, b_eadd
#pragma unroll
  for (int h = 0; h < H; ++h) {
    float v[4] = {sgy[h], sby[h], sge[h], sbe[h]};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      // over the lane groups, then the 16 lanes of a row by row moves (the
      // same pairs, quads, halves and whole row as an exchange by lane index
      // xor 1, 2, 4, 8, without an LDS round trip per step)
      const float x = row16_sum(lg_sum(v[q]));
      if (l == 0) sum_s[w][4 * h + q] = x;
    }
  }
  __syncthreads();
  // this block's slot of PS: dgamma_y [H], dbeta_y [H], db_emul [H], db_eadd [H]
  if (tid < 4 * H) {
    float x = 0.f;
#pragma unroll
    for (int ww = 0; ww < WV; ++ww) x += sum_s[ww][tid];
    const int h = tid >> 2, q = tid & 3;
    g.PS[(((size_t)b * JT + blockIdx.x) * KBZ + blockIdx.z) * 4 * H + q * H + h] = x;
  }
}

// bwd_qkv: per (head, graph, 64 output rows r0 = 64 blockIdx.z ..):
// dQ = s ds K, dK = s ds^T Q, dV = A^T dO (s the score scale) into DQKV
// [B, NP, 3, D] (float32), the contraction taken in chunks of 64 staged in
// LDS (every load of a chunk issued before any is used, out-of-range
// elements replaced by 0), products on float32 MFMA 16x16x4 tiles spread
// over the waves: lane (li, lg) supplies row li of the left operand and
// column li of the right one at contraction index 4 step + lg.
template <typename T, int H, int DH>
__global__ __launch_bounds__(kThreads) void bwd_qkv_kernel(LayerArgs a, BwdArgs g) {
  constexpr int D = H * DH, M = 64, NTN = DH / 16, TPW = 3 * 4 * NTN / kWaves;
  static_assert((3 * 4 * NTN) % kWaves == 0, "tiles over the waves");
  __shared__ float dsr_s[M][M + 1], dsc_s[M][M + 1], a_s[M][M + 1];
  __shared__ float q_s[M][DH + 1], k_s[M][DH + 1], o_s[M][DH + 1];
  const int h = blockIdx.x, b = blockIdx.y, r0 = blockIdx.z * M, NP = a.NP, n = a.n, tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, li = l & 15, lg = l >> 4;
  const size_t bh = (size_t)b * H + h;
  const T* Ag = static_cast<const T*>(g.A);
  const T* Qw = static_cast<const T*>(a.Qw);
  const T* Kw = static_cast<const T*>(a.Kw);
  const T* dO = static_cast<const T*>(g.dO);
  const int mtn = NP - r0 < M ? (NP - r0) / 16 : 4;  // 16-row tiles of this block
  f32x4 acc[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  // One contraction chunk in registers: ds rows and columns as 16-byte
  // pieces (4 per thread each), A as 2-byte values (its rows of n elements
  // are not 16-byte aligned), Q, K and dO rows as one NPD-element piece.
  // Chunk c0 + M is requested while chunk c0 is multiplied from LDS, so the
  // loads of one chunk run under the products of the previous one.
  constexpr int NPP = M * M / kThreads, NPD = M * DH / kThreads, NP4 = NPP / 4;
  struct Chunk {
    f32x4 r[NP4], c[NP4];
    uint32_t a[NPP];
    Frag<T, NPD> q, k, o;
  };
  const int prr = tid / (DH / NPD), pt0 = (tid % (DH / NPD)) * NPD;  // Q, K, dO row and column of this thread
  auto load_chunk = [&](int c0, Chunk& x) {
#pragma unroll
    for (int k = 0; k < NP4; ++k) {
      const int idx = tid + k * kThreads, hi = idx / (M / 4), lo = (idx % (M / 4)) * 4;
      // dsr: row r0 + hi, columns c0 + lo ..;  dsc: row c0 + hi, columns r0 + lo ..
      const bool okr = r0 + hi < NP && c0 + lo < NP, okc = c0 + hi < NP && r0 + lo < NP;
      x.r[k] = *reinterpret_cast<const f32x4*>(g.DS + (bh * NP + (okr ? r0 + hi : 0)) * NP + (okr ? c0 + lo : 0));
      x.c[k] = *reinterpret_cast<const f32x4*>(g.DS + (bh * NP + (okc ? c0 + hi : 0)) * NP + (okc ? r0 + lo : 0));
    }
#pragma unroll
    for (int k = 0; k < NPP; ++k) {
      const int idx = tid + k * kThreads, hi = idx / M, lo = idx % M;
      const bool oka = c0 + hi < n && r0 + lo < n;
      x.a[k] = Num<T>::ldraw(Ag + bh * n * n + (oka ? (size_t)(c0 + hi) * n + r0 + lo : 0));
    }
    const int c = c0 + prr, cp = c < NP ? c : 0, cn = c < n ? c : 0;
    x.q.load(Qw + (bh * NP + cp) * DH + pt0);
    x.k.load(Kw + (bh * NP + cp) * DH + pt0);
    x.o.load(dO + ((size_t)b * n + cn) * D + h * DH + pt0);
  };
  auto stage_chunk = [&](int c0, const Chunk& x) {
#pragma unroll
    for (int k = 0; k < NP4; ++k) {
      const int idx = tid + k * kThreads, hi = idx / (M / 4), lo = (idx % (M / 4)) * 4;
      const bool okr = r0 + hi < NP && c0 + lo < NP, okc = c0 + hi < NP && r0 + lo < NP;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dsr_s[hi][lo + e] = okr ? x.r[k][e] : 0.f;
        dsc_s[lo + e][hi] = okc ? x.c[k][e] : 0.f;  // [output row][contraction]
      }
    }
#pragma unroll
    for (int k = 0; k < NPP; ++k) {
      const int idx = tid + k * kThreads, hi = idx / M, lo = idx % M;
      a_s[lo][hi] = c0 + hi < n && r0 + lo < n ? Num<T>::fromraw(x.a[k]) : 0.f;
    }
    const int c = c0 + prr;
#pragma unroll
    for (int e = 0; e < NPD; ++e) {
      q_s[prr][pt0 + e] = c < NP ? x.q.get(e) : 0.f;
      k_s[prr][pt0 + e] = c < NP ? x.k.get(e) : 0.f;
      o_s[prr][pt0 + e] = c < n ? x.o.get(e) : 0.f;
    }
  };
  Chunk ck;
  load_chunk(0, ck);
  for (int c0 = 0; c0 < NP; c0 += M) {
    stage_chunk(c0, ck);
    __syncthreads();
    if (c0 + M < NP) load_chunk(c0 + M, ck);  // uniform
    __builtin_amdgcn_sched_barrier(0);  // the next chunk's loads stay ahead of the products
    const int csteps = (NP - c0 < M ? NP - c0 : M) / 4;
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const int ti = w + kWaves * t, which = ti / (4 * NTN), mt = (ti / NTN) % 4, nt = ti % NTN;
      if (mt >= mtn) continue;  // uniform per wave
      const int row = 16 * mt + li, col = 16 * nt + li;
      f32x4 c = acc[t];
      if constexpr (sizeof(T) == 2) {
        // bfloat16 MFMA 16x16x16 (lane (li, lg): k = 4 lg .. 4 lg + 3 of 16):
        // K, Q, A and dO are bfloat16 values, so their packing is exact;
        // the float32 ds enters as its bfloat16 rounding plus the rounded
        // remainder, a second product (2^-18 of ds per term)
#pragma unroll 2
        for (int s16 = 0; s16 < csteps / 4; ++s16) {
          const int k0 = 16 * s16 + 4 * lg;
          float av[4], bv[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            av[r] = which == 0 ? dsr_s[row][k0 + r] : which == 1 ? dsc_s[row][k0 + r] : a_s[row][k0 + r];
            bv[r] = which == 0 ? k_s[k0 + r][col] : which == 1 ? q_s[k0 + r][col] : o_s[k0 + r][col];
          }
          Frag<bf16_t, 4> ah, bq;
          ah.set(av);
          bq.set(bv);
          c = mma(c, ah, bq);
          if (which < 2) {  // uniform per wave
            float lo[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) lo[r] = av[r] - ah.get(r);
            Frag<bf16_t, 4> al;
            al.set(lo);
            c = mma(c, al, bq);
          }
        }
      } else {
#pragma unroll 4
        for (int s4 = 0; s4 < csteps; ++s4) {
          const int kk = 4 * s4 + lg;
          const float av = which == 0 ? dsr_s[row][kk] : which == 1 ? dsc_s[row][kk] : a_s[row][kk];
          const float bv = which == 0 ? k_s[kk][col] : which == 1 ? q_s[kk][col] : o_s[kk][col];
          c = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, c, 0, 0, 0);
        }
      }
      acc[t] = c;
    }
    __syncthreads();
  }
  const float sc = a.scale;
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int ti = w + kWaves * t, which = ti / (4 * NTN), mt = (ti / NTN) % 4, nt = ti % NTN;
    if (mt >= mtn) continue;
    const float f = which < 2 ? sc : 1.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int rr = r0 + 16 * mt + 4 * lg + r;
      g.DQKV[(((size_t)b * NP + rr) * 3 + which) * D + h * DH + 16 * nt + li] = f * acc[t][r];
    }
  }
}

// bwd_pair_reduce: sums over all real pairs of dgamma_e E, dbeta_e E (W_em,
// W_ea), dE' A (W_e) and dE' (b_e), as float32 MFMA contractions over the
// pairs: each block takes chunks of 64 pairs (b, i, j) in turn through LDS,
// wave w owns channels 16 w .. 16 w + 15 and keeps its partial sums in
// registers; b_e rides along as a column of ones next to the heads.
template <typename T, int H, int DE>
__global__ __launch_bounds__(kThreads) void bwd_pair_reduce_kernel(LayerArgs a, BwdArgs g) {
  constexpr int P = 64;
  static_assert(2 * H <= 16 && H < 16 && DE % 16 == 0 && DE / 16 <= kWaves, "one 16-channel chunk per wave");
  __shared__ float e_s[P][DE + 1], d_s[P][DE + 1], f_s[2 * H][P + 1], a_s[H][P + 1];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, li = l & 15, lg = l >> 4, NP = a.NP, n = a.n;
  // pair q = (b NP + i) NP + j; B NP^2 < 2^31 (checked by the library)
  const uint32_t npairs = (uint32_t)a.B * NP * NP, nchunks = (npairs + P - 1) / P;
  const T* E = static_cast<const T*>(a.E);
  const T* dEp = static_cast<const T*>(g.dEp);
  const T* Ag = static_cast<const T*>(g.A);
  f32x4 accF = {0.f, 0.f, 0.f, 0.f}, accE = {0.f, 0.f, 0.f, 0.f};
  const int cb = 16 * w;  // this wave's channels (waves past DE / 16 only help staging)
  static_assert(kThreads == 4 * P, "one thread per pair quarter");
  constexpr int NS = (P * 3 * H + kThreads - 1) / kThreads;  // dF and A values per thread
  // one chunk's loads into registers: a quarter row of E and dE' of pair
  // tid / 4, and NS of the chunk's dF / A values
  static_assert((2 * H) % 4 == 0, "dF / A rows: row w + 4 k is a dF row exactly when k < H / 2");
  struct Regs {
    Frag<T, DE / 4> ef, df;
    uint8_t mi, mj;   // mask bytes of the pair's nodes
    bool inb;         // the pair exists and both nodes are below n
    uint32_t v[NS];   // raw dF / A words (T), converted at the store
    bool inr, okv;    // pair l of the chunk exists / exists with both nodes below n
  };
  // Raw values only: the masks and bounds are applied when the chunk is
  // stored to LDS, after its loads completed.
  auto load_chunk = [&](uint32_t cidx, Regs& r) {
    {
      const int p = tid >> 2, qt = tid & 3;
      const uint32_t q = cidx * P + p;
      const uint32_t bq = q / (NP * NP), ii = (q / NP) % NP, jj = q % NP;
      const uint32_t bc = q < npairs ? bq : 0;
      r.inb = q < npairs && ii < (uint32_t)n && jj < (uint32_t)n;
      r.mi = a.mask[(size_t)bc * n + (ii < (uint32_t)n ? ii : 0)];
      r.mj = a.mask[(size_t)bc * n + (jj < (uint32_t)n ? jj : 0)];
      const size_t off = r.inb ? (((size_t)bq * n + ii) * n + jj) * DE + qt * (DE / 4) : 0;
      r.ef.load(E + off);
      r.df.load(dEp + off);
    }
    {
      const uint32_t q = cidx * P + l;  // pair l of the chunk for every k (P == 64)
      const uint32_t bq = q / (NP * NP), ii = (q / NP) % NP, jj = q % NP;
      r.inr = q < npairs;
      r.okv = r.inr && ii < (uint32_t)n && jj < (uint32_t)n;
      const uint32_t bc = r.inr ? bq : 0;  // addresses stay inside the buffers past the last pair
#pragma unroll
      for (int k = 0; k < NS; ++k) {
        const int row = w + 4 * k;  // rows 0..2H-1: dF, 2H..3H-1: A
        if (k < H / 2) {
          r.v[k] = Num<T>::ldraw(static_cast<const T*>(g.DF) + (((size_t)bc * 2 * H + row) * NP + ii) * NP + jj);
        } else {
          const int h = row < 3 * H ? row - 2 * H : 0;
          r.v[k] = Num<T>::ldraw(Ag + (((size_t)bc * H + h) * n + (r.okv ? ii : 0)) * n + (r.okv ? jj : 0));
        }
      }
    }
  };
  // one chunk: stage `cur` in LDS, load the chunk after it into `nxt`, then
  // the MFMAs; the loop alternates the two register sets (no copies)
  auto step = [&](uint32_t cidx, Regs& cur, Regs& nxt) {
    {
      const int p = tid >> 2, qt = tid & 3;
      const bool real = cur.inb && cur.mi != 0 && cur.mj != 0;
#pragma unroll
      for (int k = 0; k < DE / 4; ++k) {
        e_s[p][qt * (DE / 4) + k] = real ? cur.ef.get(k) : 0.f;
        d_s[p][qt * (DE / 4) + k] = real ? cur.df.get(k) : 0.f;
      }
#pragma unroll
      for (int k = 0; k < NS; ++k) {
        const int row = w + 4 * k;
        if (k < H / 2) f_s[row][l] = cur.inr ? Num<T>::fromraw(cur.v[k]) : 0.f;
        else if (row < 3 * H) a_s[row - 2 * H][l] = cur.okv ? Num<T>::fromraw(cur.v[k]) : 0.f;
      }
    }
    __syncthreads();
    if (cidx + gridDim.x < nchunks) load_chunk(cidx + gridDim.x, nxt);
    __builtin_amdgcn_sched_barrier(0);  // the next chunk's loads stay ahead of this chunk's MFMAs
    if (cb < DE) {
      if constexpr (sizeof(T) == 2) {
        // bfloat16: every staged value is a bfloat16 value held as a float,
        // so packing it back is exact and MFMA 16x16x16 bf16 (lane (li, lg):
        // A[li][k = 4 lg .. 4 lg + 3], B[k][li]) forms the same products as
        // the float32 form, a quarter of the MFMA issue time
#pragma unroll
        for (int k16 = 0; k16 < P / 16; ++k16) {
          const int p0 = 16 * k16 + 4 * lg;
          float fa4[4], eb4[4], da4[4], ab4[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            fa4[r] = li < 2 * H ? f_s[li < 2 * H ? li : 0][p0 + r] : 0.f;  // FiLM row li
            eb4[r] = e_s[p0 + r][cb + li];
            da4[r] = d_s[p0 + r][cb + li];
            ab4[r] = li < H ? a_s[li < H ? li : 0][p0 + r] : (li == H ? 1.f : 0.f);  // head li, or ones
          }
          Frag<bf16_t, 4> fa, eb, da, ab;
          fa.set(fa4);
          eb.set(eb4);
          da.set(da4);
          ab.set(ab4);
          accF = mma(accF, fa, eb);
          accE = mma(accE, da, ab);
        }
      } else {
        // MFMA 16x16x4: lane (li, lg) supplies A[li][k = lg] and B[k = lg][li]
#pragma unroll
        for (int ks = 0; ks < P / 4; ++ks) {
          const int pk = 4 * ks + lg;
          const float fa = li < 2 * H ? f_s[li < 2 * H ? li : 0][pk] : 0.f;  // FiLM row li
          accF = __builtin_amdgcn_mfma_f32_16x16x4f32(fa, e_s[pk][cb + li], accF, 0, 0, 0);
          const float ab = li < H ? a_s[li < H ? li : 0][pk] : (li == H ? 1.f : 0.f);  // head li, or ones
          accE = __builtin_amdgcn_mfma_f32_16x16x4f32(d_s[pk][cb + li], ab, accE, 0, 0, 0);
        }
      }
    }
    __syncthreads();
  };
  Regs r0, r1;
  if (blockIdx.x < nchunks) load_chunk(blockIdx.x, r0);
  for (uint32_t cidx = blockIdx.x; cidx < nchunks; cidx += 2 * gridDim.x) {
    step(cidx, r0, r1);
    if (cidx + gridDim.x >= nchunks) break;
    step(cidx + gridDim.x, r1, r0);
  }
  if (cb < DE) {
    // this block's row of RED: dW_emul [H][DE], dW_eadd [H][DE], dW_e [DE][H], db_e [DE]
    float* red = g.RED + (size_t)blockIdx.x * (3 * H * DE + DE);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 4 * lg + r;  // accF: FiLM row 4 lg + r, channel cb + li
      if (row < 2 * H) red[(size_t)row * DE + cb + li] = accF[r];
      const int ch = cb + 4 * lg + r;  // accE: channel cb + 4 lg + r, head li (or the sum)
      if (li < H) red[2 * H * DE + (size_t)ch * H + li] = accE[r];
      else if (li == H) red[3 * H * DE + ch] = accE[r];
    }
  }
}

// Float32 GEMM tiles for the node-level gradients (64 x 64 outputs per block,
// 32 x 32 per wave on float32 MFMA, 64-deep chunks through LDS, the next
// chunk loaded into registers while the current one is used):
//   kDX: dX[row, c] = sum_f DQKV[row, f] W_f[c] over f < 3D (W_q; W_k; W_v),
//        rows (b, i) with i < n;
//   kDW: dW_w[f, c] = sum over real rows of DQKV[row, w D + f] X[row, c],
//        and (blocks of the first column tile) db_w[f] = sum over rows of
//        DQKV[row, w D + f], read from the same staged chunks.
enum BwdGemm : int { kDX = 0, kDW = 1 };
template <typename T, int H, int DH, int MODE, int TM>
__global__ __launch_bounds__(kThreads) void bwd_gemm_kernel(LayerArgs a, BwdArgs g) {
  constexpr int D = H * DH, TN = 64, TK = 64, PERA = TK * TM / kThreads, PERB = TK * TN / kThreads;
  constexpr int MT = TM / 32;  // 16-row MFMA tiles per wave (waves in a 2 x 2 grid)
  static_assert((TM == 32 || TM == 64) && (MODE == kDX || TM == 64), "tile rows");
  __shared__ float as[TK][TM + 4], bs[TK][TN + 4];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, li = l & 15, lg = l >> 4;
  const int wm = w & 1, wn = w >> 1;
  const int m0 = blockIdx.x * TM, n0 = blockIdx.y * TN;
  const int NP = a.NP, n = a.n;
  const int M = MODE == kDX ? a.B * NP : 3 * D, K = MODE == kDX ? 3 * D : a.B * NP;
  // blockIdx.z takes a slice of the contraction (kDW: each slice writes its own partial sums)
  const int kslice = (K + gridDim.z - 1) / gridDim.z;
  const int kbeg = blockIdx.z * kslice, kend = K < kbeg + kslice ? K : kbeg + kslice;
  const T* X = static_cast<const T*>(a.X);
  // element e of this thread's share of an A chunk: kDX reads DQKV rows (k
  // fastest across the lanes), kDW reads DQKV columns (m fastest)
  auto a_kk = [&](int e) { const int idx = tid + e * kThreads; return MODE == kDX ? idx % TK : idx / TM; };
  auto a_mm = [&](int e) { const int idx = tid + e * kThreads; return MODE == kDX ? idx / TK : idx % TM; };
  // Out-of-range elements load from a clamped address and are then replaced
  // by 0: every load is issued unconditionally, so the loads of a chunk stay
  // in flight together (a load under a branch is waited for at the branch's end).
  // The replacement happens when the chunk is stored to LDS (a_ok, b_ok),
  // after its loads completed.
  auto a_ok = [&](int k0, int e) { return m0 + a_mm(e) < M && k0 + a_kk(e) < kend; };
  auto load_a = [&](int k0, int e) {
    const int m = m0 + a_mm(e), k = k0 + a_kk(e);
    const bool ok = m < M && k < kend;
    const int mc = ok ? m : 0, kc = ok ? k : 0;
    return MODE == kDX ? g.DQKV[(size_t)mc * 3 * D + kc] : g.DQKV[(size_t)kc * 3 * D + mc];
  };
  // kDW: lane l describes row k0 + l of the chunk being loaded (TK == TN ==
  // 64 == the wave size): its node's row of X (clamped), whether it is a
  // real node and its mask byte; element e of a thread lies in row
  // w + 4 e of the chunk, the same for the whole wave, read with readlane.
  static_assert(MODE == kDX || (TK == 64 && TN == 64), "one chunk row per lane");
  const int wu = __builtin_amdgcn_readfirstlane(w);
  int xr = 0;
  uint32_t mbr = 0u, okr = 0u;
  auto kdw_rows = [&](int k0) {
    const int k = k0 + l, kc = k < kend ? k : 0, bq = kc / NP, ii = kc % NP;
    xr = bq * n + (ii < n ? ii : 0);
    mbr = a.mask[(size_t)xr];
    okr = (uint32_t)(k < kend && ii < n);
  };
  // raw bits (converted at the store); kDX: a chunk lies inside one of
  // W_q, W_k, W_v (D is a multiple of TK), chosen once per chunk
  static_assert(MODE == kDW || D % TK == 0, "a chunk inside one weight");
  auto load_b = [&](int k0, int e) {
    const int idx = tid + e * kThreads, kk = idx / TN, nn = idx % TN, c = n0 + nn, k = k0 + kk;
    if (MODE == kDX) {
      const int wsel = k0 / D;
      const T* W = static_cast<const T*>(wsel == 0 ? a.w_q : wsel == 1 ? a.w_k : a.w_v);
      const bool ok = k < kend && c < D && wsel < 3;
      return Num<T>::ldraw(ok ? W + (size_t)(k - wsel * D) * D + c : static_cast<const T*>(a.w_q));
    }
    const int xrow = __builtin_amdgcn_readlane(xr, wu + 4 * e);
    return Num<T>::ldraw(X + (size_t)xrow * D + c);
  };
  // kDW: rows of padded or masked nodes count as 0 (their X may hold
  // anything); applied when the chunk is stored, after its loads completed
  auto b_ok = [&](int k0, int e) {
    if (MODE == kDX) {
      const int idx = tid + e * kThreads;
      return k0 + idx / TN < kend && n0 + idx % TN < D;
    }
    return __builtin_amdgcn_readlane(okr * mbr, wu + 4 * e) != 0u;
  };
  f32x4 acc[MT][2];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float ra[PERA];  // the next chunk, loaded while the current one is used
  uint32_t rb[PERB];
  float csum = 0.f;
  if (MODE == kDW) kdw_rows(kbeg);
#pragma unroll
  for (int e = 0; e < PERA; ++e) ra[e] = load_a(kbeg, e);
#pragma unroll
  for (int e = 0; e < PERB; ++e) rb[e] = load_b(kbeg, e);
  for (int k0 = kbeg; k0 < kend; k0 += TK) {
#pragma unroll
    for (int e = 0; e < PERA; ++e) as[a_kk(e)][a_mm(e)] = a_ok(k0, e) ? ra[e] : 0.f;
#pragma unroll
    for (int e = 0; e < PERB; ++e) {
      const int idx = tid + e * kThreads;
      bs[idx / TN][idx % TN] = b_ok(k0, e) ? Num<T>::fromraw(rb[e]) : 0.f;
    }
    __syncthreads();
    if (MODE == kDW) kdw_rows(k0 + TK);
#pragma unroll
    for (int e = 0; e < PERA; ++e) ra[e] = load_a(k0 + TK, e);
#pragma unroll
    for (int e = 0; e < PERB; ++e) rb[e] = load_b(k0 + TK, e);
    __builtin_amdgcn_sched_barrier(0);  // the next chunk's loads stay ahead of this chunk's MFMAs
    // float32 MFMA 16x16x4: wave (wm, wn) computes rows wm*TM/2 .., columns wn*32 ..
#pragma unroll
    for (int ks = 0; ks < TK / 4; ++ks) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(as[4 * ks + lg][wm * (TM / 2) + mt * 16 + li],
                                                             bs[4 * ks + lg][wn * 32 + nt * 16 + li],
                                                             acc[mt][nt], 0, 0, 0);
    }
    if (MODE == kDW && blockIdx.y == 0) {
      // bias gradients: column sums of this chunk of DQKV (all rows; rows of
      // padded or masked nodes hold 0), thread t sums rows t / 64 * TK / 4 ..
#pragma unroll
      for (int kk = 0; kk < TK / 4; ++kk) csum += as[(tid >> 6) * (TK / 4) + kk][tid & 63];
    }
    __syncthreads();
  }
  if (MODE == kDW && blockIdx.y == 0) {
    as[tid >> 6][tid & 63] = csum;
    __syncthreads();
    const int m = m0 + tid;
    if (tid < 64 && m < M) {
      const float t = as[0][tid] + as[1][tid] + as[2][tid] + as[3][tid];
      g.WP[(size_t)blockIdx.z * (3 * D * D + 3 * D) + 3 * D * D + m] = t;  // this slice's db of row m
    }
  }
#pragma unroll
  for (int e = 0; e < 8 * MT; ++e) {
    const int mt = e >> 3, nt = (e >> 2) & 1, r = e & 3;
    const int m = m0 + wm * (TM / 2) + mt * 16 + 4 * lg + r;
    if (m >= M) continue;
    {
      const int col = n0 + wn * 32 + nt * 16 + li;
      const float v = acc[mt][nt][r];
      if (col >= D) continue;
      if (MODE == kDX) {
        const int bq = m / NP, ii = m % NP;
        if (ii < n) Num<T>::st(static_cast<T*>(g.dX) + ((size_t)bq * n + ii) * D + col, v);
      } else {
        g.WP[(size_t)blockIdx.z * (3 * D * D + 3 * D) + (size_t)m * D + col] = v;  // this slice's dW
      }
    }
  }
}

// The same two GEMMs on bfloat16 MFMA (bfloat16 mode): the float32 dQ, dK,
// dV are rounded to bfloat16 (nearest even) when staged, products are
// accumulated in float32 (the projection bias sums of kDW stay float32 and
// are taken before the rounding). 64 x 64 outputs per block, 32 x 32 per
// wave on MFMA 16x16x32 bf16; chunks of 128 along the contraction are staged
// in LDS with the contraction contiguous, so each MFMA operand is one
// 16-byte LDS read (row r, contraction 8 lg .. 8 lg + 7 for lane (li, lg)).
//   kDX: rows m = (b, i) of DQKV against W_cat[k][c] = W_{k / D}[k % D][c];
//   kDW: rows f of DQKV^T against X rows (masked and padded rows count as 0).
// Staging: a thread holds 4 contraction rows x 4 columns of a source whose
// columns are contiguous, and writes each column's 4 values as one 8-byte
// LDS store (a 4 x 4 transpose in registers); kDX's DQKV rows are already
// contraction-contiguous and are written as they are.
template <int H, int DH>
__global__ __launch_bounds__(kThreads) void bwd_gemm_bf16_kernel(LayerArgs a, BwdArgs g) {
  // chunk depth TK divides D: a kDX chunk lies inside one of W_q, W_k, W_v
  constexpr int D = H * DH, TM = 64, TN = 64, TK = D >= 128 ? 128 : 64, LK = TK + 8;
  constexpr int NA = TM * TK / 4 / kThreads, NB = TN / 4 * (TK / 4) / kThreads;
  static_assert(D % 64 == 0 && D % TK == 0 && NB >= 1, "whole tiles");
  __shared__ __align__(16) uint16_t as[TM][LK];
  __shared__ __align__(16) uint16_t bs[TN][LK];
  __shared__ float cs_s[16][64];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, li = l & 15, lg = l >> 4;
  const int wm = w & 1, wn = w >> 1;
  // one launch for both products: the kDX tiles (row tile fastest), then
  // the kDW tiles (output row tile fastest, then column tile, then slice);
  // they are independent, so every block of both is resident at once
  const int nx = (a.B * a.NP + TM - 1) / TM, ndx = nx * (D / TN), nwx = 3 * D / TM;
  const int id = blockIdx.x;
  const int MODE = id < ndx ? kDX : kDW;  // uniform per block
  const int rw = id - ndx;
  const int bx = MODE == kDX ? id % nx : rw % nwx;
  const int by = MODE == kDX ? id / nx : (rw / nwx) % (D / TN);
  const int bz = MODE == kDX ? 0 : rw / (nwx * (D / TN));
  const int gz = MODE == kDX ? 1 : g.ksplit;
  const int m0 = bx * TM, n0 = by * TN;
  const int NP = a.NP, n = a.n;
  const int M = MODE == kDX ? a.B * NP : 3 * D, K = MODE == kDX ? 3 * D : a.B * NP;
  // slices of whole chunks, so that a row quad (4 rows from a multiple of 4)
  // never straddles a slice or a graph (NP is a multiple of 16)
  const int kslice = ((K + gz - 1) / gz + TK - 1) / TK * TK;
  const int kbeg = bz * kslice, kend = K < kbeg + kslice ? K : kbeg + kslice;
  const bf16_t* X = static_cast<const bf16_t*>(a.X);
  // per thread and chunk: 2 groups of (4 contraction rows x 4 columns); the
  // group's column quad cq = idx % 16 and row quad kq = idx / 16, idx = tid + 256 e
  struct Stage {
    u32x4 fa[NB][4];  // float32 source (DQKV): [group][row] 4 columns
    u32x2 hb[NB][4];  // bfloat16 source (W or X): [group][row] 4 columns
    uint8_t mk[NB][4];  // kDW: mask bytes of the X rows
    bool ok[NB][4];     // kDW: the X row exists (below kend, node below n)
  };
  // kDX's A: NA float4 per thread, rows mm = idx / (TK / 4), columns 4 (idx %
  // (TK / 4)), held in the registers of kDW's float32 source (one launch runs
  // both products, so the two share their staging registers)
  static_assert(NA == 4 * NB, "kDX's A pieces fill kDW's float32 staging");
  Stage st;
  u32x4* xa = &st.fa[0][0];
  auto load = [&](int k0) {
    if (MODE == kDX) {
      // a chunk lies wholly inside the contraction or wholly past it (the
      // prefetch after the last one, which loads chunk 0 again, unused); rows
      // m >= M load row 0 and only reach output rows that are not stored
      const int kc0 = k0 < kend ? k0 : 0, ws = kc0 / D;
#pragma unroll
      for (int e = 0; e < NA; ++e) {
        const int idx = tid + e * kThreads, m = m0 + idx / (TK / 4), mc = m < M ? m : 0;
        xa[e] = *reinterpret_cast<const u32x4*>(g.DQKV + (size_t)mc * 3 * D + kc0 + 4 * (idx % (TK / 4)));
      }
      const bf16_t* W = static_cast<const bf16_t*>(ws == 0 ? a.w_q : ws == 1 ? a.w_k : a.w_v) +
                        (size_t)(kc0 - ws * D) * D + n0;
#pragma unroll
      for (int e = 0; e < NB; ++e) {
        const int idx = tid + e * kThreads, cq = idx % 16, kq = idx / 16;
#pragma unroll
        for (int j = 0; j < 4; ++j) st.hb[e][j] = *reinterpret_cast<const u32x2*>(W + (size_t)(4 * kq + j) * D + 4 * cq);
      }
    } else {
#pragma unroll
      for (int e = 0; e < NB; ++e) {
        const int idx = tid + e * kThreads, cq = idx % 16, kq = idx / 16, r0 = k0 + 4 * kq;
        // the 4 rows r0 .. r0 + 3 lie in one graph (NP is a multiple of 16)
        const int rc = r0 < kend ? r0 : 0, bq = rc / NP, i0 = rc % NP;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bool okr = r0 + j < kend;
          st.fa[e][j] = *reinterpret_cast<const u32x4*>(g.DQKV + (size_t)(okr ? r0 + j : 0) * 3 * D + m0 + 4 * cq);
          const int i = i0 + j, ic = i < n ? i : 0;
          st.ok[e][j] = okr && i < n;
          st.mk[e][j] = a.mask[(size_t)bq * n + ic];
          st.hb[e][j] = *reinterpret_cast<const u32x2*>(X + ((size_t)bq * n + ic) * D + n0 + 4 * cq);
        }
      }
    }
  };
  float csum[4] = {0.f, 0.f, 0.f, 0.f};  // kDW bias sums of columns m0 + 4 (tid % 16) + q
  // 4 rows x 4 bfloat16 columns (u32x2 each) -> per column the 4 rows packed
  auto tr_store = [&](uint16_t (*dst)[LK], int col0, int row0, const u32x2 (&v)[4], const bool (&keep)[4]) {
    uint32_t lo[4], hi[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      lo[j] = keep[j] ? v[j].x : 0u;
      hi[j] = keep[j] ? v[j].y : 0u;
    }
    // column q is the low (q even) or high (q odd) half of word q / 2 of every
    // row; rows 2 t and 2 t + 1 share one output word (row 2 t in the low half)
    auto lo2 = [](uint32_t r0w, uint32_t r1w) { return (r0w & 0xffffu) | (r1w << 16); };
    auto hi2 = [](uint32_t r0w, uint32_t r1w) { return (r0w >> 16) | (r1w & 0xffff0000u); };
    *reinterpret_cast<u32x2*>(&dst[col0 + 0][row0]) = u32x2{lo2(lo[0], lo[1]), lo2(lo[2], lo[3])};
    *reinterpret_cast<u32x2*>(&dst[col0 + 1][row0]) = u32x2{hi2(lo[0], lo[1]), hi2(lo[2], lo[3])};
    *reinterpret_cast<u32x2*>(&dst[col0 + 2][row0]) = u32x2{lo2(hi[0], hi[1]), lo2(hi[2], hi[3])};
    *reinterpret_cast<u32x2*>(&dst[col0 + 3][row0]) = u32x2{hi2(hi[0], hi[1]), hi2(hi[2], hi[3])};
  };
  auto store = [&](int k0) {
    if (MODE == kDX) {
#pragma unroll
      for (int e = 0; e < NA; ++e) {
        const int idx = tid + e * kThreads, mm = idx / (TK / 4), kk = 4 * (idx % (TK / 4));
        const u32x4 v = xa[e];
        *reinterpret_cast<u32x2*>(&as[mm][kk]) =
            u32x2{pack_bf2(__uint_as_float(v.x), __uint_as_float(v.y)), pack_bf2(__uint_as_float(v.z), __uint_as_float(v.w))};
      }
      const bool keep[4] = {true, true, true, true};
#pragma unroll
      for (int e = 0; e < NB; ++e) {
        const int idx = tid + e * kThreads, cq = idx % 16, kq = idx / 16;
        tr_store(bs, 4 * cq, 4 * kq, st.hb[e], keep);
      }
    } else {
#pragma unroll
      for (int e = 0; e < NB; ++e) {
        const int idx = tid + e * kThreads, cq = idx % 16, kq = idx / 16;
        bool keep[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) keep[j] = st.ok[e][j] && st.mk[e][j] != 0;
        tr_store(bs, 4 * cq, 4 * kq, st.hb[e], keep);
        // DQKV^T: columns f = m0 + 4 cq + q, rows 4 kq + j (float32 -> bfloat16)
        float f[4][4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bool okr = k0 + 4 * kq + j < kend;
          f[j][0] = okr ? __uint_as_float(st.fa[e][j].x) : 0.f;
          f[j][1] = okr ? __uint_as_float(st.fa[e][j].y) : 0.f;
          f[j][2] = okr ? __uint_as_float(st.fa[e][j].z) : 0.f;
          f[j][3] = okr ? __uint_as_float(st.fa[e][j].w) : 0.f;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          csum[q] += (f[0][q] + f[1][q]) + (f[2][q] + f[3][q]);
          *reinterpret_cast<u32x2*>(&as[4 * cq + q][4 * kq]) = u32x2{pack_bf2(f[0][q], f[1][q]), pack_bf2(f[2][q], f[3][q])};
        }
      }
    }
  };
  f32x4 acc[2][2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  load(kbeg);
  for (int k0 = kbeg; k0 < kend; k0 += TK) {
    store(k0);
    __syncthreads();
    load(k0 + TK);
    __builtin_amdgcn_sched_barrier(0);  // the next chunk's loads stay ahead of this chunk's MFMAs
#pragma unroll
    for (int ks = 0; ks < TK / 32; ++ks) {
      u32x4 af[2], bf[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        af[t] = *reinterpret_cast<const u32x4*>(&as[wm * 32 + t * 16 + li][32 * ks + 8 * lg]);
        bf[t] = *reinterpret_cast<const u32x4*>(&bs[wn * 32 + t * 16 + li][32 * ks + 8 * lg]);
      }
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, af[mt]),
                                                                __builtin_bit_cast(bf16x8, bf[nt]), acc[mt][nt], 0, 0, 0);
    }
    __syncthreads();
  }
  if (MODE == kDW && by == 0) {
    // bias sums: the 16 threads of a column quad (tid % 16) reduce through LDS
#pragma unroll
    for (int q = 0; q < 4; ++q) cs_s[tid / 16][4 * (tid % 16) + q] = csum[q];
    __syncthreads();
    if (tid < 64 && m0 + tid < M) {
      float t = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) t += cs_s[r][tid];
      g.WP[(size_t)bz * (3 * D * D + 3 * D) + 3 * D * D + m0 + tid] = t;  // this slice's db
    }
  }
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int mt = e >> 3, nt = (e >> 2) & 1, r = e & 3;
    const int m = m0 + wm * 32 + mt * 16 + 4 * lg + r, col = n0 + wn * 32 + nt * 16 + li;
    if (m >= M) continue;
    const float v = acc[mt][nt][r];
    if (MODE == kDX) {
      const int bq = m / NP, ii = m % NP;
      if (ii < n) Num<bf16_t>::st(static_cast<bf16_t*>(g.dX) + ((size_t)bq * n + ii) * D + col, v);
    } else {
      g.WP[(size_t)bz * (3 * D * D + 3 * D) + (size_t)m * D + col] = v;  // this slice's dW
    }
  }
}

// bwd_sums: the fixed-order sums of the partial slots (no atomics anywhere
// in the backward, so every run gives the same bits). Blocks, in order:
//   B blocks, one per graph: DGY[b] = sum over the pair kernel's blocks of
//     the graph (PS rows in order): dgamma_y, dbeta_y, and the graph's parts
//     of db_emul, db_eadd;
//   ceil(NR / 16) blocks of 16 columns of RED (NR = 3 H de + de): dW_emul,
//     dW_eadd, dW_e, db_e as sums over the pair reduction's rows;
//   then one thread per projection gradient (dW_q|k|v, db_q|k|v): the sum
//     over the dW GEMM's contraction slices.
// Column sums take a fixed split of the rows over the threads and add the
// threads' parts in a fixed order.
template <typename T, int H, int DH, int DE>
__global__ __launch_bounds__(kThreads) void bwd_sums_kernel(LayerArgs a, BwdArgs g) {
  constexpr int NR = 3 * H * DE + DE, F = 4 * H, CB = 16, D = H * DH;
  __shared__ __align__(16) float part_s[4 * kThreads];
  const int tid = threadIdx.x, B = a.B;
  const int nrb = (NR + CB - 1) / CB;
  if ((int)blockIdx.x < B) {
    // the graph's PS rows: F columns as F / 4 16-byte column groups, the
    // rows split over kThreads / (F / 4) row groups (rows q, q + RG2, ...),
    // each thread's rows loaded 16 at a time, the row groups added in order
    constexpr int CG = F / 4, RG2 = kThreads / CG, U = 16;
    static_assert(F % 4 == 0 && kThreads % CG == 0 && RG2 * F <= 4 * kThreads, "column groups");
    const int b = blockIdx.x, rows = a.NP / 16 * g.ps_kb;
    const int cg = tid % CG, q = tid / CG;
    const float* base = g.PS + (size_t)b * rows * F + 4 * cg;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    int r = q;
    for (; r + (U - 1) * RG2 < rows; r += U * RG2) {
      f32x4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = *reinterpret_cast<const f32x4*>(base + (size_t)(r + u * RG2) * F);
#pragma unroll
      for (int u = 0; u < U; ++u) acc += v[u];
    }
    for (; r < rows; r += RG2) acc += *reinterpret_cast<const f32x4*>(base + (size_t)r * F);
    *reinterpret_cast<f32x4*>(&part_s[q * F + 4 * cg]) = acc;
    __syncthreads();
    if (tid < F) {
      float t = 0.f;
      for (int k = 0; k < RG2; ++k) t += part_s[k * F + tid];
      g.DGY[(size_t)b * F + tid] = t;
    }
  } else if ((int)blockIdx.x < B + nrb) {
    // 16 columns as four 16-byte column groups; the rows split over 64 row
    // groups (rows q, q + 64, ...), each thread's rows loaded 16 at a time
    static_assert(NR % CB == 0 && CB == 16, "whole 16-byte column groups");
    constexpr int RG = kThreads / 4, U = 16;
    const int cg = tid & 3, q = tid >> 2, c0 = ((int)blockIdx.x - B) * CB + 4 * cg;
    const float* base = g.RED + c0;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const int rows = g.red_rows;
    int r = q;
    for (; r + (U - 1) * RG < rows; r += U * RG) {
      f32x4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = *reinterpret_cast<const f32x4*>(base + (size_t)(r + u * RG) * NR);
#pragma unroll
      for (int u = 0; u < U; ++u) acc += v[u];
    }
    for (; r < rows; r += RG) acc += *reinterpret_cast<const f32x4*>(base + (size_t)r * NR);
    *reinterpret_cast<f32x4*>(&part_s[4 * tid]) = acc;
    __syncthreads();
    if (tid < CB) {
      const int c = ((int)blockIdx.x - B) * CB + tid;
      float t = 0.f;
      for (int k = 0; k < RG; ++k) t += part_s[16 * k + tid];  // row group k holds columns 4 cg .. of its 4 threads
      if (c < H * DE) g.gw_em[c] = t;
      else if (c < 2 * H * DE) g.gw_ea[c - H * DE] = t;
      else if (c < 3 * H * DE) g.gw_e[c - 2 * H * DE] = t;
      else g.gb_e[c - 3 * H * DE] = t;
    }
  } else {
    const size_t nw = (size_t)3 * D * D + 3 * D;
    const size_t o = (size_t)((int)blockIdx.x - B - nrb) * kThreads + tid;
    if (o >= nw) return;
    // every slice's value requested at once (clamped slice index, the surplus
    // discarded by a uniform condition), then added in slice order
    float v[kMaxKsplit];
#pragma unroll
    for (int z = 0; z < kMaxKsplit; ++z) v[z] = g.WP[(size_t)(z < g.ksplit ? z : g.ksplit - 1) * nw + o];
    float t = 0.f;
#pragma unroll
    for (int z = 0; z < kMaxKsplit; ++z)
      if (z < g.ksplit) t += v[z];
    if (o < (size_t)3 * D * D) {
      const int wsel = (int)(o / ((size_t)D * D));
      (wsel == 0 ? g.gw_q : wsel == 1 ? g.gw_k : g.gw_v)[o % ((size_t)D * D)] = t;
    } else {
      const int m = (int)(o - (size_t)3 * D * D), wsel = m / D;
      (wsel == 0 ? g.gb_q : wsel == 1 ? g.gb_k : g.gb_v)[m % D] = t;
    }
  }
}

// bwd_small: the global FiLM's gradients and dy, from the per-graph sums
// DGY [B, 4H] (dgamma_y, dbeta_y, db_emul part, db_eadd part); one thread
// per item, sums over the graphs in graph order:
//   dy[b][c]         = sum_h W_ymul[h][c] dgamma_y[b][h] + W_yadd[h][c] dbeta_y[b][h]
//   dW_y(mul|add)[h][c] = sum_b dgamma_y|dbeta_y[b][h] y[b][c]
//   db_y(mul|add)[h]    = sum_b dgamma_y|dbeta_y[b][h]
//   db_e(mul|add)[h]    = sum_b (the graph's part)
template <typename T, int H, int DH, int DE>
__global__ __launch_bounds__(kThreads) void bwd_small_kernel(LayerArgs a, BwdArgs g) {
  constexpr int F = 4 * H;
  const int B = a.B, dy = a.dy;
  const int item = blockIdx.x * kThreads + threadIdx.x;
  const int n_dy = B * dy, n_w = 2 * H * dy, n_b = 2 * H;
  const T* y = static_cast<const T*>(a.y);
  const T* Wm = static_cast<const T*>(a.w_ymul);
  const T* Wa = static_cast<const T*>(a.w_yadd);
  // sum over the graphs of DGY[b][o] times f(b), graph b into partial sum
  // b % 4 in graph order; sixteen graphs' loads per step, then four
  auto over_graphs = [&](int o, auto f) {
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    int b = 0;
    for (; b + 15 < B; b += 16) {
      float v[16], w[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        v[u] = g.DGY[(size_t)(b + u) * F + o];
        w[u] = f(b + u);
      }
#pragma unroll
      for (int u = 0; u < 16; ++u) acc[u & 3] += v[u] * w[u];
    }
    for (; b + 3 < B; b += 4) {
      float v[4], w[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        v[u] = g.DGY[(size_t)(b + u) * F + o];
        w[u] = f(b + u);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) acc[u] += v[u] * w[u];
    }
    for (; b < B; ++b) acc[0] += g.DGY[(size_t)b * F + o] * f(b);
    return (acc[0] + acc[1]) + (acc[2] + acc[3]);
  };
  if (item < n_dy) {
    const int b = item / dy, c = item % dy;
    float dg[2 * H], wv[2 * H];
#pragma unroll
    for (int o = 0; o < 2 * H; ++o) {
      dg[o] = g.DGY[(size_t)b * F + o];
      wv[o] = Num<T>::ld((o < H ? Wm : Wa) + (size_t)(o % H) * dy + c);
    }
    float s = 0.f;
#pragma unroll
    for (int o = 0; o < 2 * H; ++o) s += wv[o] * dg[o];
    Num<T>::st(static_cast<T*>(g.dy) + (size_t)b * dy + c, s);
  } else if (item < n_dy + n_w) {
    const int o = (item - n_dy) / dy, c = (item - n_dy) % dy;
    const float s = over_graphs(o, [&](int b) { return Num<T>::ld(y + (size_t)b * dy + c); });
    (o < H ? g.gw_ym : g.gw_ya)[(size_t)(o % H) * dy + c] = s;
  } else if (item < n_dy + n_w + n_b) {
    const int o = item - n_dy - n_w;
    (o < H ? g.gb_ym : g.gb_ya)[o % H] = over_graphs(o, [](int) { return 1.f; });
  } else if (item < n_dy + n_w + 2 * n_b) {
    const int o = item - n_dy - n_w - n_b;  // 0 .. 2H - 1: db_emul, then db_eadd
    (o < H ? g.gb_em : g.gb_ea)[o % H] = over_graphs(2 * H + o, [](int) { return 1.f; });
  }
}

// ------------------------------------------------------------------ dispatch

// Compute units of the current device (queried once per device).
int num_cus() {
  static int cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cached[dev]) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    cached[dev] = v;
  }
  return cached[dev];
}


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
    case kFused:
      if constexpr (sizeof(T) == 2 && DE == 64) {
        // two or three key tiles per wave: E streamed through LDS
        // (fused_stream_kernel; with four, its K and V fragments would not
        // fit in registers)
        switch (maxt) {
          case 2: hipLaunchKernelGGL((fused_stream_kernel<T, H, DH, DE, 2>), grid, dim3(kThreads), 0, s, a); return hipGetLastError();
          case 3: hipLaunchKernelGGL((fused_stream_kernel<T, H, DH, DE, 3>), grid, dim3(kThreads), 0, s, a); return hipGetLastError();
          default: break;
        }
      }
      return attn_maxt<T, H, DH, DE, kFused>(a, maxt, grid, s);
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
  const dim3 grid((unsigned)JT * ((JT + kWaves - 1) / kWaves), a.B);  // < 2^31 for n <= 2^20
  if constexpr (sizeof(T) == 2 && DE % 32 == 0) {
    if (mode == kRecompute || mode == kRecomputeU) {
      // persistent pipeline: one block per compute unit, items = grid of the plain kernel
      const int items = (int)grid.x * (int)grid.y;  // B NP/16 ceil(NP/64) < 2^31 for n <= 2^20
      const int blocks = items < num_cus() ? items : num_cus();
      if (mode == kRecompute)
        hipLaunchKernelGGL((update_pipe_kernel<T, H, DH, DE, kRecompute>), dim3(blocks), dim3(kThreads), 0, s, a, items);
      else
        hipLaunchKernelGGL((update_pipe_kernel<T, H, DH, DE, kRecomputeU>), dim3(blocks), dim3(kThreads), 0, s, a, items);
      return hipGetLastError();
    }
  }
  if (mode == kReadA)
    hipLaunchKernelGGL((update_kernel<T, H, DH, DE, kReadA>), grid, dim3(kThreads), 0, s, a);
  else if (mode == kRecompute)
    hipLaunchKernelGGL((update_kernel<T, H, DH, DE, kRecompute>), grid, dim3(kThreads), 0, s, a);
  else if (mode == kRecomputeU)
    hipLaunchKernelGGL((update_kernel<T, H, DH, DE, kRecomputeU>), grid, dim3(kThreads), 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

template <typename T, int D, int DH>
hipError_t qkv_shape(const LayerArgs& a, hipStream_t s) {
  const long rows = (long)a.B * a.NP;
  // one extra column of blocks computes the global FiLM coefficients
  const dim3 grid((unsigned)((rows + 63) / 64), 3 * D / 64 + 1 + (a.order ? 1 : 0));  // rows < 2^31
  hipLaunchKernelGGL((qkv_kernel<T, D, DH>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <typename T, int H, int DH, int DE>
hipError_t backward_shape(const LayerArgs& a, const BwdArgs& g0, hipStream_t s) {
  constexpr int D = H * DH;
  const int JT = a.NP / 16;
  BwdArgs g = g0;
  const size_t chunks = ((size_t)a.B * a.NP * a.NP + 63) / 64;
  // the pair reduction: 1024 blocks, four per CU (the LDS fits four), all resident
  g.red_rows = (int)(chunks < (size_t)kRedRows ? chunks : (size_t)kRedRows);
  // dW: the rows (contraction) split in slices of at least 256
  const int rows = a.B * a.NP;
  g.ksplit = rows / 256 < 1 ? 1 : (rows / 256 > kMaxKsplit ? kMaxKsplit : rows / 256);
  // n > 64 and two-pass: the second pair pass runs kUseSplit blocks per 64
  // keys, each with its own slot of the per-block sums
  constexpr int kUseWaves = kWaves / kUseSplit;
  static_assert(kUseWaves * kUseSplit == kWaves, "whole key tiles per block");
  g.ps_kb = (g.recompute_a || a.NP > 64) ? kUseSplit * ((a.NP + 63) / 64) : 1;
  const unsigned prep_blocks = (unsigned)((size_t)a.B * H * ((a.NP + 63) / 64));  // < 2^31 for n <= 2^20
  hipLaunchKernelGGL((bwd_prep_kernel<T, H, DH, DE>), dim3(prep_blocks), dim3(kThreads), 0, s, a, g);
  const int KB = (a.NP + 63) / 64;
  if (g.recompute_a) {  // two-pass context: A recomputed (and stored) by the first pass
    hipLaunchKernelGGL((bwd_pair_kernel<T, H, DH, DE, kPairPartA>), dim3(JT, a.B, KB), dim3(kThreads), 0, s, a, g);
    hipLaunchKernelGGL((bwd_pair_kernel<T, H, DH, DE, kPairUse, kUseWaves>), dim3(JT, a.B, kUseSplit * KB), dim3(64 * kUseWaves), 0, s, a, g);
  } else if (a.NP <= 64) {
    hipLaunchKernelGGL((bwd_pair_kernel<T, H, DH, DE, kPairAll>), dim3(JT, a.B, 1), dim3(kThreads), 0, s, a, g);
  } else {  // key blocks of 64: the row sums of D first, then the rest
    hipLaunchKernelGGL((bwd_pair_kernel<T, H, DH, DE, kPairPart>), dim3(JT, a.B, KB), dim3(kThreads), 0, s, a, g);
    hipLaunchKernelGGL((bwd_pair_kernel<T, H, DH, DE, kPairUse, kUseWaves>), dim3(JT, a.B, kUseSplit * KB), dim3(64 * kUseWaves), 0, s, a, g);
  }
  hipLaunchKernelGGL((bwd_qkv_kernel<T, H, DH>), dim3(H, a.B, (a.NP + 63) / 64), dim3(kThreads), 0, s, a, g);
  hipLaunchKernelGGL((bwd_pair_reduce_kernel<T, H, DE>), dim3(g.red_rows), dim3(kThreads), 0, s, a, g);
  const dim3 gdx((a.B * a.NP + 63) / 64, D / 64, 1), gdw(3 * D / 64, D / 64, g.ksplit);
  if constexpr (sizeof(T) == 2) {
    // both products in one launch: the kDX tiles, then the kDW tiles
    const unsigned nboth = gdx.x * gdx.y + gdw.x * gdw.y * gdw.z;
    hipLaunchKernelGGL((bwd_gemm_bf16_kernel<H, DH>), dim3(nboth), dim3(kThreads), 0, s, a, g);
  } else {
    hipLaunchKernelGGL((bwd_gemm_kernel<T, H, DH, kDX, 64>), gdx, dim3(kThreads), 0, s, a, g);
    hipLaunchKernelGGL((bwd_gemm_kernel<T, H, DH, kDW, 64>), gdw, dim3(kThreads), 0, s, a, g);
  }
  constexpr int NR = 3 * H * DE + DE;
  const size_t sums_blocks = (size_t)a.B + (NR + 15) / 16 + ((size_t)3 * D * D + 3 * D + kThreads - 1) / kThreads;
  hipLaunchKernelGGL((bwd_sums_kernel<T, H, DH, DE>), dim3((unsigned)sums_blocks), dim3(kThreads), 0, s, a, g);
  const size_t small_items = (size_t)a.B * a.dy + 2 * H * a.dy + 4 * H;
  hipLaunchKernelGGL((bwd_small_kernel<T, H, DH, DE>), dim3((unsigned)((small_items + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, s, a, g);
  return hipGetLastError();
}

}  // namespace

bool wants_order(int dtype, int H, int dh, int de, int B, int NP) {
  // fused_stream_kernel: bfloat16, de = 64, two or three key tiles per wave
  const int JT = NP / 16, maxt = (JT + kWaves - 1) / kWaves;
  return dtype == 1 && shape_supported(dtype, H, dh, de) && de == 64 && (maxt == 2 || maxt == 3) &&
         (long)B * JT <= kOrderMax;
}

bool shape_supported(int dtype, int H, int dh, int de) {
  if (dtype != 0 && dtype != 1) return false;
  return (H == 4 && dh == 16 && de == 16) || (H == 8 && dh == 32 && de == 64);
}

#define EA_SHAPES(CALL, T)                                          \
  if (H == 4 && dh == 16 && de == 16) return CALL(T, 4, 16, 16);    \
  if (H == 8 && dh == 32 && de == 64) return CALL(T, 8, 32, 64);

hipError_t launch_backward(const LayerArgs& a, const BwdArgs& g, int dtype, int H, int dh, int de,
                           hipStream_t s) {
  // float32 edge tiles of de = 64 do not fit in registers next to the rest
  // of the pair kernel: float32 is built for the (4, 16, 16) shape only
  if (dtype == 1 && H == 4 && dh == 16 && de == 16) return backward_shape<bf16_t, 4, 16, 16>(a, g, s);
  if (dtype == 1 && H == 8 && dh == 32 && de == 64) return backward_shape<bf16_t, 8, 32, 64>(a, g, s);
  if (dtype == 0 && H == 4 && dh == 16 && de == 16) return backward_shape<float, 4, 16, 16>(a, g, s);
  return hipErrorInvalidValue;
}

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
