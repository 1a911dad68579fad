// C ABI of the edge-aware attention layer: argument validation, workspace
// plan, mode choice (one pass or the two-pass scheme for large graphs) and
// kernel launches on the caller's stream.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <new>
#include <algorithm>
#include <mutex>
#include <vector>

#include "edge_attn.h"
#include "ea_internal.h"

struct ea_ctx {
  ea_desc d;
  int NP;          // n rounded up to a multiple of 16
  int two_pass;
  int generic;     // the shape has no tuned kernels: the generic path runs
  int forward_done;
  const void* a_written;  // two-pass: the A buffer the last edge_attn_layer call filled (else NULL)
  size_t esz;      // element size of desc.dtype
  size_t off_q, off_k, off_v, off_lse, off_gy, off_order, ws_bytes;
  size_t boff_ds, boff_df, boff_dqkv, boff_dgy, boff_ps, boff_red, boff_wp, boff_dp, boff_ar, bws_bytes;  // backward workspace
  int blk_nxb, blk_exb;  // block: node and edge blocks per graph
  size_t blk_off_o, blk_off_a, blk_off_px, blk_off_pe, blk_bytes;  // block workspace (after the layer's)
  // kernel timing window
  int prof_on;
  std::vector<hipEvent_t> ev_pool;
  std::vector<int> ev_kernel;  // kernel id of each recorded pair
  size_t ev_used;
};

namespace {

thread_local char g_err[512] = "";

ea_status fail(ea_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

ea_status check_ptr(const void* p, const char* name, size_t align, bool required) {
  if (!p) return required ? fail(EA_E_NULLPTR, "%s is NULL", name) : EA_OK;
  if (!aligned(p, align)) return fail(EA_E_ALIGN, "%s is not %zu-byte aligned", name, align);
  return EA_OK;
}

#define EA_TRY(x)                 \
  do {                            \
    ea_status s_ = (x);           \
    if (s_ != EA_OK) return s_;   \
  } while (0)

constexpr uint32_t kVariants = EA_VARIANT_LIGHT_EDGE | EA_VARIANT_NO_SCORE_MOD | EA_VARIANT_UNNORMALIZED;

bool edge_film_on(const ea_ctx* c) {
  return (c->d.flags & (EA_VARIANT_LIGHT_EDGE | EA_VARIANT_NO_SCORE_MOD)) == 0;
}
bool global_film_on(const ea_ctx* c) { return (c->d.flags & EA_VARIANT_NO_SCORE_MOD) == 0; }
bool unnormalized(const ea_ctx* c) { return (c->d.flags & EA_VARIANT_UNNORMALIZED) != 0; }

// FiLM parameters the variant does not read may be NULL.
ea_status check_attn_params(const ea_ctx* c, const ea_attn_params* p) {
  if (!p) return fail(EA_E_NULLPTR, "attention parameters are NULL");
  EA_TRY(check_ptr(p->w_q, "w_q", 16, true));
  EA_TRY(check_ptr(p->w_k, "w_k", 16, true));
  EA_TRY(check_ptr(p->w_v, "w_v", 16, true));
  EA_TRY(check_ptr(p->w_emul, "w_emul", 16, edge_film_on(c)));
  EA_TRY(check_ptr(p->w_eadd, "w_eadd", 16, edge_film_on(c)));
  EA_TRY(check_ptr(p->w_ymul, "w_ymul", 4, global_film_on(c)));
  EA_TRY(check_ptr(p->w_yadd, "w_yadd", 4, global_film_on(c)));
  EA_TRY(check_ptr(p->b_q, "b_q", 4, false));
  EA_TRY(check_ptr(p->b_k, "b_k", 4, false));
  EA_TRY(check_ptr(p->b_v, "b_v", 4, false));
  EA_TRY(check_ptr(p->b_emul, "b_emul", 4, false));
  EA_TRY(check_ptr(p->b_eadd, "b_eadd", 4, false));
  EA_TRY(check_ptr(p->b_ymul, "b_ymul", 4, false));
  EA_TRY(check_ptr(p->b_yadd, "b_yadd", 4, false));
  return EA_OK;
}

ea_status check_ws(const ea_ctx* c, void* ws, size_t ws_bytes) {
  if (!ws) return fail(EA_E_WORKSPACE, "workspace is NULL (%zu bytes required)", c->ws_bytes);
  if (!aligned(ws, 256)) return fail(EA_E_ALIGN, "workspace is not 256-byte aligned");
  if (ws_bytes < c->ws_bytes)
    return fail(EA_E_WORKSPACE, "workspace has %zu bytes, %zu required", ws_bytes, c->ws_bytes);
  return EA_OK;
}

ea::LayerArgs make_args(const ea_ctx* c, const ea_attn_params* p, const ea_update_params* u,
                        const void* X, const void* E, const void* y, const uint8_t* mask,
                        void* ws) {
  ea::LayerArgs a;
  memset(&a, 0, sizeof(a));
  a.X = X; a.E = E; a.y = y; a.mask = mask;
  if (p) {
    a.w_q = p->w_q; a.w_k = p->w_k; a.w_v = p->w_v;
    a.b_q = p->b_q; a.b_k = p->b_k; a.b_v = p->b_v;
    a.w_emul = p->w_emul; a.w_eadd = p->w_eadd; a.b_emul = p->b_emul; a.b_eadd = p->b_eadd;
    a.w_ymul = p->w_ymul; a.w_yadd = p->w_yadd; a.b_ymul = p->b_ymul; a.b_yadd = p->b_yadd;
  }
  if (u) { a.w_e = u->w_e; a.b_e = u->b_e; }
  char* base = static_cast<char*>(ws);
  a.Qw = base + c->off_q;
  a.Kw = base + c->off_k;
  a.Vt = base + c->off_v;
  a.lse = reinterpret_cast<float*>(base + c->off_lse);
  a.gy = reinterpret_cast<float*>(base + c->off_gy);
  a.B = c->d.B; a.n = c->d.n; a.NP = c->NP; a.dy = c->d.dy;
  a.H = c->d.H; a.dh = c->d.dh; a.de = c->d.de; a.d = c->d.d;
  a.scale = (float)(1.0 / sqrt((double)c->d.dh));
  a.variant = (int)(c->d.flags & kVariants);
  return a;
}

// Launch with optional event timing around it.
template <typename F>
ea_status timed(ea_ctx* c, int kernel, hipStream_t s, F&& launch) {
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (c->prof_on && c->ev_used + 2 <= c->ev_pool.size()) {
    e0 = c->ev_pool[c->ev_used];
    e1 = c->ev_pool[c->ev_used + 1];
    c->ev_kernel.push_back(kernel);
    c->ev_used += 2;
    if (hipEventRecord(e0, s) != hipSuccess) return fail(EA_E_HIP, "hipEventRecord failed");
  }
  hipError_t err = launch();
  if (err != hipSuccess)
    return fail(EA_E_HIP, "%s launch failed: %s", ea_kernel_name(kernel), hipGetErrorString(err));
  if (e1 && hipEventRecord(e1, s) != hipSuccess) return fail(EA_E_HIP, "hipEventRecord failed");
  return EA_OK;
}

ea_status run_qkv(ea_ctx* c, const ea::LayerArgs& a, hipStream_t s) {
  if (c->generic) return timed(c, EA_K_QKV, s, [&] { return ea::launch_gen_qkv(a, c->d.dtype, s); });
  return timed(c, EA_K_QKV, s, [&] { return ea::launch_qkv(a, c->d.dtype, c->d.H, c->d.dh, c->d.de, s); });
}

// The generic path's row kernel (every shape the boundary accepts).
ea_status run_gen(ea_ctx* c, const ea::LayerArgs& a, int kernel, int mode, hipStream_t s) {
  return timed(c, kernel, s, [&] { return ea::launch_gen_row(a, c->d.dtype, mode, c->two_pass, s); });
}

ea_status check_io(const ea_ctx* c, const void* X, const void* E, const void* y,
                   const uint8_t* mask, bool needX) {
  if (needX) EA_TRY(check_ptr(X, "X", 16, true));
  EA_TRY(check_ptr(E, "E", 16, true));
  EA_TRY(check_ptr(y, "y", 4, global_film_on(c)));
  if (!mask) return fail(EA_E_NULLPTR, "node_mask is NULL");
  return EA_OK;
}

// Workspace of edge_attn_layer_noalloc: a file-scope device array, so that
// the call allocates nothing. Each GPU the library runs on holds its own
// copy until the process ends. In host code the array's name is not a device
// address; the address of this device's copy comes from hipGetSymbolAddress
// (once per device, with that device current) and only that address is used.
constexpr size_t kScratchBytes = size_t(16) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

ea_status scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(EA_E_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(EA_E_HIP, "device %d is beyond the %d supported", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(EA_E_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return EA_OK;
}

}  // namespace

extern "C" {

const char* ea_status_str(ea_status s) {
  switch (s) {
    case EA_OK: return "ok";
    case EA_E_NULLPTR: return "null pointer";
    case EA_E_SHAPE: return "bad shape";
    case EA_E_UNSUPPORTED: return "unsupported configuration";
    case EA_E_ALIGN: return "misaligned pointer";
    case EA_E_WORKSPACE: return "workspace too small";
    case EA_E_STATE: return "call order violated";
    case EA_E_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* ea_last_error(void) { return g_err; }

const char* ea_kernel_name(int k) {
  switch (k) {
    case EA_K_QKV: return "qkv_kernel";
    case EA_K_ATTN: return "attn_kernel";
    case EA_K_UPDATE: return "update_kernel";
    case EA_K_FUSED: return "attn_kernel(fused)";
    case EA_K_BACKWARD: return "backward (all kernels)";
    case EA_K_BLOCK: return "block (node, edge, y kernels)";
  }
  return "?";
}

ea_status ea_ctx_create(const ea_desc* desc, ea_ctx** out) {
  g_err[0] = 0;
  if (!desc || !out) return fail(EA_E_NULLPTR, "desc or out is NULL");
  *out = nullptr;
  const ea_desc& d = *desc;
  if (d.B < 1 || d.n < 1 || d.d < 1 || d.de < 1 || d.dy < 1 || d.H < 1 || d.dh < 1)
    return fail(EA_E_SHAPE, "all sizes must be >= 1 (B=%d n=%d d=%d de=%d dy=%d H=%d dh=%d)",
                d.B, d.n, d.d, d.de, d.dy, d.H, d.dh);
  if ((long long)d.H * d.dh != d.d) return fail(EA_E_SHAPE, "d (%d) != H*dh (%d*%d)", d.d, d.H, d.dh);
  if (d.B > 65535) return fail(EA_E_SHAPE, "B (%d) exceeds 65535", d.B);
  if (d.n > (1 << 20)) return fail(EA_E_SHAPE, "n (%d) exceeds 2^20", d.n);
  if ((long long)d.B * ((d.n + 15) / 16 * 16) >= (1ll << 31))
    return fail(EA_E_SHAPE, "B * n (padded to 16) must stay below 2^31");
  if (d.dtype != EA_FP32 && d.dtype != EA_BF16) return fail(EA_E_UNSUPPORTED, "dtype %d", d.dtype);
  if (d.flags & ~(EA_FORCE_TWO_PASS | kVariants)) return fail(EA_E_UNSUPPORTED, "unknown flags 0x%x", d.flags);
  if (d.dh != 16 && d.dh != 32 && d.dh != 64)
    return fail(EA_E_UNSUPPORTED, "dh = %d: the head width must be 16, 32 or 64", d.dh);
  if (d.de % 16 != 0) return fail(EA_E_UNSUPPORTED, "de = %d: the edge width must be a multiple of 16", d.de);
  if (2 * d.H > 32) return fail(EA_E_UNSUPPORTED, "H = %d: at most 16 heads (2H <= 32)", d.H);
  if ((long long)d.B * d.n * d.n * d.de >= (1ll << 46))
    return fail(EA_E_SHAPE, "the edge tensor B n^2 de must stay below 2^46 elements");
  ea_ctx* c = new (std::nothrow) ea_ctx();
  if (!c) return fail(EA_E_SHAPE, "out of host memory");
  c->d = d;
  c->NP = (d.n + 15) / 16 * 16;
  c->two_pass = (d.flags & EA_FORCE_TWO_PASS) || d.n > EA_SINGLE_PASS_MAX_N;
  c->generic = !ea::shape_supported(d.dtype, d.H, d.dh, d.de);
  c->forward_done = 0;
  c->a_written = nullptr;
  c->esz = d.dtype == EA_BF16 ? 2 : 4;
  const size_t qkv = round256((size_t)d.B * d.H * c->NP * d.dh * c->esz);
  c->off_q = 0;
  c->off_k = qkv;
  c->off_v = 2 * qkv;
  c->off_lse = 3 * qkv;
  c->off_gy = c->off_lse + round256((size_t)d.B * d.H * c->NP * sizeof(float));
  c->off_order = c->off_gy + round256((size_t)d.B * 2 * d.H * sizeof(float));
  c->ws_bytes = c->off_order + round256((size_t)d.B * (c->NP / 16) * sizeof(int));
  const size_t pairs = (size_t)d.B * c->NP * c->NP;
  c->boff_ds = qkv;  // V rows first
  c->boff_df = c->boff_ds + round256(pairs * d.H * sizeof(float));
  c->boff_dqkv = c->boff_df + round256(pairs * 2 * d.H * c->esz);
  c->boff_dgy = c->boff_dqkv + round256((size_t)d.B * c->NP * 3 * d.d * sizeof(float));
  c->boff_ps = c->boff_dgy + round256((size_t)d.B * 4 * d.H * sizeof(float));
  c->boff_red = c->boff_ps + round256((size_t)d.B * (c->NP / 16) * (ea::kUseSplit * ((c->NP + 63) / 64)) * 4 * d.H * sizeof(float));
  c->boff_wp = c->boff_red + round256((size_t)ea::kRedRows * (3 * d.H * d.de + d.de) * sizeof(float));
  c->boff_dp = c->boff_wp + round256((size_t)ea::kMaxKsplit * (3 * (size_t)d.d * d.d + 3 * d.d) * sizeof(float));
  c->boff_ar = c->boff_dp + round256((size_t)d.B * d.H * c->NP * ((c->NP + 63) / 64) * sizeof(float));
  // two-pass contexts: the backward recomputes A [B, H, n, n] into its workspace
  c->bws_bytes = c->boff_ar + (c->two_pass ? round256((size_t)d.B * d.H * d.n * d.n * c->esz) : 0);
  {
    // block: 16 nodes per node block; edge blocks of 4 waves with at least
    // 4 tiles of 16 tokens per wave, at most 256 per graph
    const size_t tiles = ((size_t)d.n * d.n + 15) / 16;
    c->blk_nxb = (d.n + 15) / 16;
    c->blk_exb = (int)std::min<size_t>(256, std::max<size_t>(1, (tiles + 15) / 16));
    c->blk_off_o = c->ws_bytes;
    c->blk_off_a = c->blk_off_o + round256((size_t)d.B * d.n * d.d * c->esz);
    c->blk_off_px = c->blk_off_a + (c->two_pass ? 0 : round256((size_t)d.B * d.H * d.n * d.n * c->esz));
    c->blk_off_pe = c->blk_off_px + round256((size_t)d.B * c->blk_nxb * d.d * sizeof(float));
    c->blk_bytes = c->blk_off_pe + round256((size_t)d.B * c->blk_exb * d.de * sizeof(float));
  }
  c->prof_on = 0;
  c->ev_used = 0;
  *out = c;
  return EA_OK;
}

void ea_ctx_destroy(ea_ctx* c) {
  if (!c) return;
  for (hipEvent_t e : c->ev_pool) (void)hipEventDestroy(e);
  delete c;
}

size_t ea_workspace_bytes(const ea_ctx* c) { return c ? c->ws_bytes : 0; }

int ea_is_two_pass(const ea_ctx* c) { return c ? c->two_pass : -1; }

ea_status edge_attn_forward(ea_ctx* c, const ea_attn_params* p, const void* X, const void* E,
                            const void* y, const uint8_t* mask, void* O, void* A, void* ws,
                            size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  if (!c) return fail(EA_E_NULLPTR, "ctx is NULL");
  EA_TRY(check_attn_params(c, p));
  EA_TRY(check_io(c, X, E, y, mask, true));
  EA_TRY(check_ptr(O, "O", 16, true));
  if (c->two_pass) {
    if (A) return fail(EA_E_UNSUPPORTED, "A is not produced in two-pass mode; pass NULL");
  } else {
    EA_TRY(check_ptr(A, "A", 16, true));
  }
  EA_TRY(check_ws(c, ws, ws_bytes));
  hipStream_t s = static_cast<hipStream_t>(stream);
  ea::LayerArgs a = make_args(c, p, nullptr, X, E, y, mask, ws);
  a.O = O;
  a.A = A;
  c->forward_done = 0;
  c->a_written = nullptr;
  EA_TRY(run_qkv(c, a, s));
  if (c->generic) {
    EA_TRY(run_gen(c, a, EA_K_ATTN, ea::kGenForward, s));
    c->forward_done = 1;
    return EA_OK;
  }
  const int mode = c->two_pass ? ea::kOnline : ea::kSingle;
  EA_TRY(timed(c, EA_K_ATTN, s, [&] { return ea::launch_attn(a, c->d.dtype, c->d.H, c->d.dh, c->d.de, mode, s); }));
  c->forward_done = 1;
  return EA_OK;
}

// The edge update; A_out (two-pass, no variant flag): the second pass also
// writes the attention map it recomputes.
static ea_status update_impl(ea_ctx* c, const ea_attn_params* p, const ea_update_params* u,
                             const void* E, const void* y, const uint8_t* mask, const void* A,
                             void* A_out, void* E_out, void* ws, size_t ws_bytes, void* stream) {
  if (!c) return fail(EA_E_NULLPTR, "ctx is NULL");
  if (!u) return fail(EA_E_NULLPTR, "update parameters are NULL");
  EA_TRY(check_ptr(u->w_e, "w_e", 16, true));
  EA_TRY(check_ptr(u->b_e, "b_e", 4, false));
  EA_TRY(check_ptr(E_out, "E_out", 16, true));
  EA_TRY(check_ptr(E, "E", 16, true));
  if (!mask) return fail(EA_E_NULLPTR, "node_mask is NULL");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (c->two_pass || unnormalized(c)) {
    // the update recomputes the logits from E and the forward's workspace
    EA_TRY(check_attn_params(c, p));
    EA_TRY(check_ptr(y, "y", 4, global_film_on(c)));
    EA_TRY(check_ws(c, ws, ws_bytes));
    if (!c->forward_done)
      return fail(EA_E_STATE, "%s edge_update needs a preceding edge_attn_forward on this context",
                  c->two_pass ? "two-pass" : "unnormalized-variant");
    ea::LayerArgs a = make_args(c, p, u, nullptr, E, y, mask, ws);
    a.E_out = E_out;
    a.A = A_out;
    if (c->generic) return run_gen(c, a, EA_K_UPDATE, ea::kGenUpdate, s);
    const int mode = unnormalized(c) ? ea::kRecomputeU : ea::kRecompute;
    return timed(c, EA_K_UPDATE, s, [&] {
      return ea::launch_update(a, c->d.dtype, c->d.H, c->d.dh, c->d.de, mode, s);
    });
  }
  EA_TRY(check_ptr(A, "A", 16, true));
  ea::LayerArgs a = make_args(c, nullptr, u, nullptr, E, y, mask, ws ? ws : E_out);
  a.A = const_cast<void*>(A);
  a.E_out = E_out;
  if (c->generic) return run_gen(c, a, EA_K_UPDATE, ea::kGenUpdate, s);
  return timed(c, EA_K_UPDATE, s, [&] {
    return ea::launch_update(a, c->d.dtype, c->d.H, c->d.dh, c->d.de, ea::kReadA, s);
  });
}

ea_status edge_update(ea_ctx* c, const ea_attn_params* p, const ea_update_params* u,
                      const void* E, const void* y, const uint8_t* mask, const void* A,
                      void* E_out, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  return update_impl(c, p, u, E, y, mask, A, nullptr, E_out, ws, ws_bytes, stream);
}

ea_status edge_attn_layer(ea_ctx* c, const ea_attn_params* p, const ea_update_params* u,
                          const void* X, const void* E, const void* y, const uint8_t* mask,
                          void* O, void* A, void* E_out, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  if (!c) return fail(EA_E_NULLPTR, "ctx is NULL");
  if (c->two_pass || unnormalized(c)) {
    if (c->generic) {  // one row kernel: both passes and the update
      if (!u) return fail(EA_E_NULLPTR, "update parameters are NULL");
      EA_TRY(check_ptr(u->w_e, "w_e", 16, true));
      EA_TRY(check_ptr(u->b_e, "b_e", 4, false));
      EA_TRY(check_ptr(E_out, "E_out", 16, true));
      EA_TRY(check_attn_params(c, p));
      EA_TRY(check_io(c, X, E, y, mask, true));
      EA_TRY(check_ptr(O, "O", 16, true));
      if (c->two_pass && A) return fail(EA_E_UNSUPPORTED, "A is not produced in two-pass mode; pass NULL");
      if (!c->two_pass) EA_TRY(check_ptr(A, "A", 16, true));
      EA_TRY(check_ws(c, ws, ws_bytes));
      hipStream_t s = static_cast<hipStream_t>(stream);
      ea::LayerArgs a = make_args(c, p, u, X, E, y, mask, ws);
      a.O = O; a.A = A; a.E_out = E_out;
      c->forward_done = 0;
      c->a_written = nullptr;
      EA_TRY(run_qkv(c, a, s));
      EA_TRY(run_gen(c, a, EA_K_FUSED, ea::kGenLayer, s));
      c->forward_done = 1;
      return EA_OK;
    }
    // Validate everything before the first launch.
    if (!u) return fail(EA_E_NULLPTR, "update parameters are NULL");
    EA_TRY(check_ptr(u->w_e, "w_e", 16, true));
    EA_TRY(check_ptr(u->b_e, "b_e", 4, false));
    EA_TRY(check_ptr(E_out, "E_out", 16, true));
    if (!c->two_pass) {  // unnormalized variant, one pass: A from the forward, the update recomputes
      EA_TRY(edge_attn_forward(c, p, X, E, y, mask, O, A, ws, ws_bytes, stream));
      return update_impl(c, p, u, E, y, mask, nullptr, nullptr, E_out, ws, ws_bytes, stream);
    }
    // two-pass: A, if given, is written by the second pass
    if (A && unnormalized(c))
      return fail(EA_E_UNSUPPORTED, "A is not produced by the two-pass scheme with the unnormalized variant");
    EA_TRY(check_ptr(A, "A", 16, false));
    EA_TRY(edge_attn_forward(c, p, X, E, y, mask, O, nullptr, ws, ws_bytes, stream));
    EA_TRY(update_impl(c, p, u, E, y, mask, nullptr, A, E_out, ws, ws_bytes, stream));
    c->a_written = A;
    return EA_OK;
  }
  EA_TRY(check_attn_params(c, p));
  EA_TRY(check_io(c, X, E, y, mask, true));
  EA_TRY(check_ptr(O, "O", 16, true));
  EA_TRY(check_ptr(A, "A", 16, true));
  if (!u) return fail(EA_E_NULLPTR, "update parameters are NULL");
  EA_TRY(check_ptr(u->w_e, "w_e", 16, true));
  EA_TRY(check_ptr(u->b_e, "b_e", 4, false));
  EA_TRY(check_ptr(E_out, "E_out", 16, true));
  EA_TRY(check_ws(c, ws, ws_bytes));
  hipStream_t s = static_cast<hipStream_t>(stream);
  ea::LayerArgs a = make_args(c, p, u, X, E, y, mask, ws);
  a.O = O;
  a.A = A;
  a.E_out = E_out;
  if (!c->generic && !c->two_pass && ea::wants_order(c->d.dtype, c->d.H, c->d.dh, c->d.de, c->d.B, c->NP))
    a.order = reinterpret_cast<int*>(static_cast<char*>(ws) + c->off_order);
  c->forward_done = 0;
  c->a_written = nullptr;
  EA_TRY(run_qkv(c, a, s));
  if (c->generic) {
    EA_TRY(run_gen(c, a, EA_K_FUSED, ea::kGenLayer, s));
    c->forward_done = 1;
    return EA_OK;
  }
  EA_TRY(timed(c, EA_K_FUSED, s, [&] {
    return ea::launch_attn(a, c->d.dtype, c->d.H, c->d.dh, c->d.de, ea::kFused, s);
  }));
  c->forward_done = 1;
  return EA_OK;
}

size_t ea_noalloc_max_workspace_bytes(void) { return kScratchBytes; }

ea_status edge_attn_layer_noalloc(ea_ctx* c, const ea_attn_params* p, const ea_update_params* u,
                                  const void* X, const void* E, const void* y, const uint8_t* mask,
                                  void* O, void* A, void* E_out, void* stream) {
  g_err[0] = 0;
  if (!c) return fail(EA_E_NULLPTR, "ctx is NULL");
  if (c->ws_bytes > kScratchBytes)
    return fail(EA_E_WORKSPACE, "the layer needs %zu bytes of workspace; edge_attn_layer_noalloc holds at most %zu",
                c->ws_bytes, kScratchBytes);
  void* ws = nullptr;
  EA_TRY(scratch_address(&ws));
  const ea_status st = edge_attn_layer(c, p, u, X, E, y, mask, O, A, E_out, ws, kScratchBytes, stream);
  // the workspace is internal and shared by later calls: no backward or
  // two-pass edge_update may rely on what this call left in it
  c->forward_done = 0;
  c->a_written = nullptr;
  return st;
}

ea_status ea_debug_logits(ea_ctx* c, const ea_attn_params* p, const void* X, const void* E,
                          const void* y, const uint8_t* mask, float* U, void* ws, size_t ws_bytes,
                          void* stream) {
  g_err[0] = 0;
  if (!c) return fail(EA_E_NULLPTR, "ctx is NULL");
  EA_TRY(check_attn_params(c, p));
  EA_TRY(check_io(c, X, E, y, mask, true));
  EA_TRY(check_ptr(U, "U", 16, true));
  EA_TRY(check_ws(c, ws, ws_bytes));
  if (!c->generic && c->NP > 4 * 64)
    return fail(EA_E_UNSUPPORTED, "the tuned logit export is limited to n <= 256");
  hipStream_t s = static_cast<hipStream_t>(stream);
  ea::LayerArgs a = make_args(c, p, nullptr, X, E, y, mask, ws);
  a.U = U;
  EA_TRY(run_qkv(c, a, s));
  if (c->generic) return run_gen(c, a, EA_K_ATTN, ea::kGenLogits, s);
  return timed(c, EA_K_ATTN, s, [&] {
    return ea::launch_attn(a, c->d.dtype, c->d.H, c->d.dh, c->d.de, ea::kLogits, s);
  });
}

ea_status ea_debug_softmax(ea_ctx* c, const float* U, void* A, void* stream) {
  g_err[0] = 0;
  if (!c) return fail(EA_E_NULLPTR, "ctx is NULL");
  EA_TRY(check_ptr(U, "U", 16, true));
  EA_TRY(check_ptr(A, "A", 16, true));
  const long rows = (long)c->d.B * c->d.H * c->d.n;
  if (rows >= (1l << 31)) return fail(EA_E_SHAPE, "B H n must stay below 2^31");
  hipStream_t s = static_cast<hipStream_t>(stream);
  return timed(c, EA_K_ATTN, s, [&] { return ea::launch_gen_softmax(U, A, rows, c->d.n, c->d.dtype, s); });
}

ea_status ea_probe_copy(const void* src, void* dst, size_t bytes, void* stream) {
  g_err[0] = 0;
  if (bytes == 0) return EA_OK;
  EA_TRY(check_ptr(src, "src", 16, true));
  EA_TRY(check_ptr(dst, "dst", 16, true));
  if (bytes % 16) return fail(EA_E_ALIGN, "bytes must be a multiple of 16");
  const hipError_t e = ea::launch_probe_copy(src, dst, bytes / 16, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? EA_OK : fail(EA_E_HIP, "probe copy launch failed: %s", hipGetErrorString(e));
}

ea_status ea_probe_read(const void* src, size_t bytes, uint32_t* xor_out, void* stream) {
  g_err[0] = 0;
  EA_TRY(check_ptr(src, "src", 16, bytes > 0));
  EA_TRY(check_ptr(xor_out, "xor_out", 4, true));
  if (bytes % 16) return fail(EA_E_ALIGN, "bytes must be a multiple of 16");
  const hipError_t e = ea::launch_probe_read(src, bytes / 16, xor_out, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? EA_OK : fail(EA_E_HIP, "probe read launch failed: %s", hipGetErrorString(e));
}

size_t ea_block_workspace_bytes(const ea_ctx* c) { return c ? c->blk_bytes : 0; }

ea_status edge_attn_block(ea_ctx* c, const ea_attn_params* p, const ea_update_params* u,
                          const ea_block_params* bp, const void* X, const void* E, const void* y,
                          const uint8_t* mask, void* X_out, void* E_out, void* y_out,
                          void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  if (!c) return fail(EA_E_NULLPTR, "ctx is NULL");
  if (c->d.flags & kVariants) return fail(EA_E_UNSUPPORTED, "the block is built for the full layer (no variant flag)");
  if (!ea::block_supported(c->d.dtype == EA_BF16 ? 1 : 0, c->d.d, c->d.de, c->d.dy))
    return fail(EA_E_UNSUPPORTED, "the block is built for (d, de, dy) = (64, 16, 16) and, in bfloat16, (256, 64, 64)");
  if (!bp) return fail(EA_E_NULLPTR, "block parameters are NULL");
  const void* const* bpp = reinterpret_cast<const void* const*>(bp);
  static_assert(sizeof(ea_block_params) == ea::kBlockParams * sizeof(void*), "block parameter list");
  static const char* const kNames[ea::kBlockParams] = {
      "w_o", "b_o", "ln_x1_g", "ln_x1_b", "w_x1", "b_x1", "w_x2", "b_x2", "ln_x2_g", "ln_x2_b",
      "ln_e1_g", "ln_e1_b", "w_e1", "b_e1", "w_e2", "b_e2", "ln_e2_g", "ln_e2_b",
      "w_yy", "w_yx", "w_ye", "b_yo", "ln_y1_g", "ln_y1_b", "w_y1", "b_y1", "w_y2", "b_y2", "ln_y2_g", "ln_y2_b"};
  for (int q = 0; q < ea::kBlockParams; ++q) EA_TRY(check_ptr(bpp[q], kNames[q], 16, true));
  EA_TRY(check_attn_params(c, p));
  EA_TRY(check_io(c, X, E, y, mask, true));
  if (!y) return fail(EA_E_NULLPTR, "y is NULL (the block updates it)");
  EA_TRY(check_ptr(X_out, "X_out", 16, true));
  EA_TRY(check_ptr(E_out, "E_out", 16, true));
  EA_TRY(check_ptr(y_out, "y_out", 4, true));
  if (!u) return fail(EA_E_NULLPTR, "update parameters are NULL");
  EA_TRY(check_ptr(u->w_e, "w_e", 16, true));
  EA_TRY(check_ptr(u->b_e, "b_e", 4, false));
  if (!ws) return fail(EA_E_WORKSPACE, "workspace is NULL (%zu bytes required)", c->blk_bytes);
  if (!aligned(ws, 256)) return fail(EA_E_WORKSPACE, "workspace must be 256-byte aligned");
  if (ws_bytes < c->blk_bytes)
    return fail(EA_E_WORKSPACE, "block workspace has %zu bytes, %zu required", ws_bytes, c->blk_bytes);
  char* wb = static_cast<char*>(ws);
  void* O = wb + c->blk_off_o;
  void* A = c->two_pass ? nullptr : wb + c->blk_off_a;
  EA_TRY(edge_attn_layer(c, p, u, X, E, y, mask, O, A, E_out, ws, c->ws_bytes, stream));
  ea::BlockArgs k;
  memset(&k, 0, sizeof(k));
  for (int q = 0; q < ea::kBlockParams; ++q) k.p[q] = bpp[q];
  k.X = X; k.y = y; k.mask = mask; k.O = O; k.E_io = E_out; k.X_out = X_out; k.y_out = y_out;
  k.part_x = reinterpret_cast<float*>(wb + c->blk_off_px);
  k.part_e = reinterpret_cast<float*>(wb + c->blk_off_pe);
  k.B = c->d.B; k.n = c->d.n; k.dy = c->d.dy; k.nxb = c->blk_nxb; k.exb = c->blk_exb;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return timed(c, EA_K_BLOCK, s, [&] { return ea::launch_block(k, c->d.dtype, c->d.d, c->d.de, s); });
}

size_t ea_backward_workspace_bytes(const ea_ctx* c) { return c ? c->bws_bytes : 0; }

ea_status edge_attn_backward(ea_ctx* c, const ea_attn_params* p, const ea_update_params* u,
                             const void* X, const void* E, const void* y, const uint8_t* mask,
                             const void* A, const void* dO, const void* dEp,
                             void* dX, void* dE, void* dy, const ea_grads* gr,
                             void* ws, size_t ws_bytes, void* bws, size_t bws_bytes, void* stream) {
  g_err[0] = 0;
  if (!c) return fail(EA_E_NULLPTR, "ctx is NULL");
  if ((uint64_t)c->d.B * c->NP * c->NP >= (1ull << 31))
    return fail(EA_E_UNSUPPORTED, "the backward indexes pairs in 32 bits: B n_p^2 must stay below 2^31");
  if (c->d.flags & kVariants) return fail(EA_E_UNSUPPORTED, "the backward is built for the full layer (no variant flag)");
  if (c->generic)
    return fail(EA_E_UNSUPPORTED, "the backward is built for (H, dh, de) = (4, 16, 16) and (8, 32, 64)");
  if (c->d.dtype == EA_FP32 && c->d.de != 16)
    return fail(EA_E_UNSUPPORTED, "the float32 backward is built for (H, dh, de) = (4, 16, 16)");
  EA_TRY(check_attn_params(c, p));
  EA_TRY(check_ptr(p->b_emul, "b_emul", 4, false));
  if (!u) return fail(EA_E_NULLPTR, "update parameters are NULL");
  EA_TRY(check_ptr(u->w_e, "w_e", 16, true));
  EA_TRY(check_ptr(u->b_e, "b_e", 4, false));
  EA_TRY(check_io(c, X, E, y, mask, true));
  EA_TRY(check_ptr(A, "A", 16, !c->two_pass));  // two-pass: used only if the preceding layer call wrote it
  EA_TRY(check_ptr(dO, "dO", 16, true));
  EA_TRY(check_ptr(dEp, "dE_out", 16, true));
  EA_TRY(check_ptr(dX, "dX", 16, true));
  EA_TRY(check_ptr(dE, "dE", 16, true));
  EA_TRY(check_ptr(dy, "dy", 4, true));
  if (!gr) return fail(EA_E_NULLPTR, "grads is NULL");
  const void* gp[] = {gr->w_q, gr->w_k, gr->w_v, gr->b_q, gr->b_k, gr->b_v, gr->w_emul, gr->w_eadd,
                      gr->b_emul, gr->b_eadd, gr->w_ymul, gr->w_yadd, gr->b_ymul, gr->b_yadd, gr->w_e, gr->b_e};
  for (const void* q : gp) EA_TRY(check_ptr(q, "a gradient buffer", 16, true));
  EA_TRY(check_ws(c, ws, ws_bytes));
  if (!bws) return fail(EA_E_WORKSPACE, "backward workspace is NULL (%zu bytes required)", c->bws_bytes);
  if (!aligned(bws, 256)) return fail(EA_E_ALIGN, "backward workspace is not 256-byte aligned");
  if (bws_bytes < c->bws_bytes)
    return fail(EA_E_WORKSPACE, "backward workspace has %zu bytes, %zu required", bws_bytes, c->bws_bytes);
  if (!c->forward_done)
    return fail(EA_E_STATE, "edge_attn_backward needs a preceding forward on this context");
  hipStream_t s = static_cast<hipStream_t>(stream);
  ea::LayerArgs a = make_args(c, p, u, X, E, y, mask, ws);
  ea::BwdArgs g;
  memset(&g, 0, sizeof(g));
  g.A = A; g.dO = dO; g.dEp = dEp; g.dX = dX; g.dE = dE; g.dy = dy;
  g.gw_q = gr->w_q; g.gw_k = gr->w_k; g.gw_v = gr->w_v; g.gb_q = gr->b_q; g.gb_k = gr->b_k; g.gb_v = gr->b_v;
  g.gw_em = gr->w_emul; g.gw_ea = gr->w_eadd; g.gb_em = gr->b_emul; g.gb_ea = gr->b_eadd;
  g.gw_ym = gr->w_ymul; g.gw_ya = gr->w_yadd; g.gb_ym = gr->b_ymul; g.gb_ya = gr->b_yadd;
  g.gw_e = gr->w_e; g.gb_e = gr->b_e;
  char* bb = static_cast<char*>(bws);
  g.Vr = bb;
  g.DS = reinterpret_cast<float*>(bb + c->boff_ds);
  g.DF = bb + c->boff_df;
  g.DQKV = reinterpret_cast<float*>(bb + c->boff_dqkv);
  g.DGY = reinterpret_cast<float*>(bb + c->boff_dgy);
  g.PS = reinterpret_cast<float*>(bb + c->boff_ps);
  g.RED = reinterpret_cast<float*>(bb + c->boff_red);
  g.WP = reinterpret_cast<float*>(bb + c->boff_wp);
  g.DP = reinterpret_cast<float*>(bb + c->boff_dp);
  if (c->two_pass && !(A && A == c->a_written)) {  // A recomputed from the logits and lse into the workspace
    g.A = bb + c->boff_ar;
    g.recompute_a = 1;
  }
  return timed(c, EA_K_BACKWARD, s, [&] {
    return ea::launch_backward(a, g, c->d.dtype, c->d.H, c->d.dh, c->d.de, s);
  });
}

ea_status ea_profile_begin(ea_ctx* c) {
  g_err[0] = 0;
  if (!c) return fail(EA_E_NULLPTR, "ctx is NULL");
  const size_t want = 2 * 4096;
  while (c->ev_pool.size() < want) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return fail(EA_E_HIP, "hipEventCreate failed");
    c->ev_pool.push_back(e);
  }
  c->ev_kernel.clear();
  c->ev_used = 0;
  c->prof_on = 1;
  return EA_OK;
}

ea_status ea_profile_end(ea_ctx* c, double* total_ms, int64_t* launches) {
  g_err[0] = 0;
  if (!c) return fail(EA_E_NULLPTR, "ctx is NULL");
  if (!total_ms || !launches) return fail(EA_E_NULLPTR, "output arrays are NULL");
  for (int k = 0; k < EA_NUM_KERNELS; ++k) { total_ms[k] = 0.0; launches[k] = 0; }
  c->prof_on = 0;
  if (c->ev_used && hipEventSynchronize(c->ev_pool[c->ev_used - 1]) != hipSuccess)
    return fail(EA_E_HIP, "hipEventSynchronize failed");
  for (size_t k = 0; k < c->ev_kernel.size(); ++k) {
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, c->ev_pool[2 * k], c->ev_pool[2 * k + 1]) != hipSuccess)
      return fail(EA_E_HIP, "hipEventElapsedTime failed");
    total_ms[c->ev_kernel[k]] += ms;
    launches[c->ev_kernel[k]] += 1;
  }
  c->ev_kernel.clear();
  c->ev_used = 0;
  return EA_OK;
}

}  // extern "C"
