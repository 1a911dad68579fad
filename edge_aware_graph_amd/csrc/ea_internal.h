// Internal interface between the C-ABI host code and the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ea {

// Kernel modes of the attention kernel.
enum AttnMode : int {
  kSingle = 0,  // one pass over full rows: writes O and A
  kFused = 1,   // kSingle plus the residual edge update: writes O, A and E'
  kOnline = 2,  // two-pass pass 1: online softmax, writes O and softmax statistics
  kLogits = 3,  // stage export: writes the masked logits u
};
// Kernel modes of the edge-update kernel.
enum UpdateMode : int {
  kReadA = 0,       // single pass: A comes from the forward's output
  kRecompute = 1,   // two-pass pass 2: A = exp(u - lse) recomputed per tile
  kRecomputeU = 2,  // unnormalized variant: the operand is the logit u itself
};
// Ablation variant bits (LayerArgs::variant); the same values as the
// EA_VARIANT_* flags of the C ABI.
enum Variant : int {
  kLightEdge = 0x2,     // no per-edge FiLM: gamma_e = 1, beta_e = 0
  kNoScoreMod = 0x4,    // no FiLM at all: u = s
  kUnnormalized = 0x8,  // the edge update takes u (0 at masked pairs) instead of A
};

struct LayerArgs {
  // inputs
  const void* X;
  const void* E;
  const void* y;
  const uint8_t* mask;
  const void *w_q, *w_k, *w_v, *b_q, *b_k, *b_v;
  const void *w_emul, *w_eadd, *b_emul, *b_eadd;
  const void *w_ymul, *w_yadd, *b_ymul, *b_yadd;
  const void *w_e, *b_e;
  // workspace
  void* Qw;    // [B, H, NP, dh]
  void* Kw;    // [B, H, NP, dh]
  void* Vt;    // [B, H, dh, NP]
  float* lse;  // [B, H, NP]
  float* gy;   // [B, 2H]: gamma_y (1 + ...) then beta_y per graph
  int* order;  // [B NP/16]: work order of the layer's attention kernel, or NULL (see wants_order)
  // outputs
  void* O;
  void* A;       // attention map (kSingle/kFused) or the map to read (kReadA)
  void* E_out;
  float* U;      // logits (kLogits)
  // sizes
  int B, n, NP, dy;
  int H, dh, de, d;  // runtime copies (the tuned kernels take them as template parameters)
  float scale;   // 1/sqrt(dh)
  int variant;   // Variant bits
};

// Backward of one layer (single pass, n <= 64): gradients and scratch.
struct BwdArgs {
  const void* A;    // the forward's attention map [B, H, n, n]
  const void* dO;   // loss gradient of O [B, n, d]
  const void* dEp;  // loss gradient of E' [B, n, n, de]
  void* dX;         // [B, n, d]
  void* dE;         // [B, n, n, de]
  void* dy;         // [B, dy]
  float *gw_q, *gw_k, *gw_v, *gb_q, *gb_k, *gb_v;  // float32 weight gradients
  float *gw_em, *gw_ea, *gb_em, *gb_ea;
  float *gw_ym, *gw_ya, *gb_ym, *gb_ya;
  float *gw_e, *gb_e;
  // scratch (the backward workspace)
  void* Vr;      // V rows [B, H, NP, dh]
  float* DS;     // ds [B, H, NP, NP] (float32: the key-bias gradient, a sum of ds over keys, nearly cancels)
  void* DF;      // dgamma_e, dbeta_e [B, 2H, NP, NP], the layer's dtype
  float* DQKV;   // dQ | dK | dV [B, NP, 3, d]
  float* DGY;    // per graph: dgamma_y, dbeta_y, and the graph's parts of db_emul, db_eadd [B, 4H]
  float* PS;     // the same four sums per block of the pair kernel [B, NP / 16, ps_kb, 4H]
  float* RED;    // pair-reduction sums, one row per block of the reduction [red_rows][2 H de + de H + de]
  float* WP;     // dW GEMM: weight and bias gradients per contraction slice [ksplit][3 d d + 3 d]
  float* DP;     // n > 64: parts of D_i = sum_j A_ij dA_ij per key block [B, H, NP, ceil(NP / 64)]
  int recompute_a;  // two-pass context: A [B, H, n, n] is recomputed into the buffer g.A points to
  int ps_kb;        // key blocks of the pair-kernel launch that writes PS
  int red_rows;     // blocks of the pair reduction
  int ksplit;       // contraction slices of the dW GEMM
};

// The backward sums nothing with atomics: every block writes its partial
// sums to a slot of its own and a later kernel adds the slots in a fixed
// order, so the gradients are the same bits on every run.
constexpr int kRedRows = 1024;  // most blocks of the pair reduction
constexpr int kMaxKsplit = 16;  // most contraction slices of the dW GEMM
// blocks per 64 keys in the backward's second pair pass (n > 64 or two-pass
// contexts): blocks of two waves (32 keys), two to a CU, so that their phases
// need not coincide; each block writes its own slot of the per-block sums
constexpr int kUseSplit = 2;

// Graph-transformer block around the layer: parameters (in this order; the
// nn.Linear [out, in] layout, all in the layer's dtype) and arguments.
enum BlockParam : int {
  kBW_o, kBb_o, kBln_x1_g, kBln_x1_b, kBW_x1, kBb_x1, kBW_x2, kBb_x2, kBln_x2_g, kBln_x2_b,
  kBln_e1_g, kBln_e1_b, kBW_e1, kBb_e1, kBW_e2, kBb_e2, kBln_e2_g, kBln_e2_b,
  kBW_yy, kBW_yx, kBW_ye, kBb_yo, kBln_y1_g, kBln_y1_b, kBW_y1, kBb_y1, kBW_y2, kBb_y2, kBln_y2_g, kBln_y2_b,
  kBlockParams
};
struct BlockArgs {
  const void* p[kBlockParams];
  const void* X;          // [B, n, d]
  const void* y;          // [B, dy]
  const uint8_t* mask;    // [B, n]
  const void* O;          // the layer's node output [B, n, d]
  void* E_io;             // E' in, E2 out [B, n, n, de]
  void* X_out;            // [B, n, d]
  void* y_out;            // [B, dy]
  float* part_x;          // [B, nxb, d] sums of X2 over real nodes per node block
  float* part_e;          // [B, exb, de] sums of E2 over real pairs per edge block
  int B, n, dy, nxb, exb;
};
bool block_supported(int dtype, int d, int de, int dy);
hipError_t launch_block(const BlockArgs& k, int dtype, int d, int de, hipStream_t s);

// Launchers; each returns the hipError_t of its launch. `dtype` 0 = fp32, 1 = bf16.
hipError_t launch_qkv(const LayerArgs& a, int dtype, int H, int dh, int de, hipStream_t s);
hipError_t launch_attn(const LayerArgs& a, int dtype, int H, int dh, int de, int mode,
                       hipStream_t s);
hipError_t launch_update(const LayerArgs& a, int dtype, int H, int dh, int de, int mode,
                         hipStream_t s);
// The backward's kernels in order (prep, pair, per-head, pair reduction,
// dX, dW, small sums); returns the first launch error.
hipError_t launch_backward(const LayerArgs& a, const BwdArgs& g, int dtype, int H, int dh, int de,
                           hipStream_t s);
// Bandwidth probes (ea_probe.hip): a plain copy of n16 16-byte pieces, and a
// plain read whose words are XOR-ed into *xor_out.
hipError_t launch_probe_copy(const void* src, void* dst, size_t n16, hipStream_t s);
hipError_t launch_probe_read(const void* src, size_t n16, uint32_t* xor_out, hipStream_t s);
// Whether (dtype, H, dh, de) is instantiated.
bool shape_supported(int dtype, int H, int dh, int de);
// Whether the layer's attention kernel (kFused) for this shape takes a work
// order (LayerArgs::order), which qkv_kernel then writes.
bool wants_order(int dtype, int H, int dh, int de, int B, int NP);

// Generic path: any shape the boundary accepts (dh in {16, 32, 64}, de a
// multiple of 16, 2H <= 32), one block per query row, runtime sizes.
enum GenMode : int {
  kGenForward = 0,  // O, and A (single pass) or lse (two-pass)
  kGenLayer = 1,    // O, A (single pass) and E'
  kGenUpdate = 2,   // E' from A (single pass) or from A recomputed with lse (two-pass)
  kGenLogits = 3,   // the masked logits u
};
hipError_t launch_gen_qkv(const LayerArgs& a, int dtype, hipStream_t s);
hipError_t launch_gen_row(const LayerArgs& a, int dtype, int mode, int two_pass, hipStream_t s);
// Row softmax of float32 logits U [rows, n] into A [rows, n] (layer dtype).
hipError_t launch_gen_softmax(const float* U, void* A, long rows, int n, int dtype, hipStream_t s);

}  // namespace ea
