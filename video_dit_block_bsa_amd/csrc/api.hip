// C ABI of libbsa.so (declared in include/bsa.h): argument checks, workspace
// layout and kernel dispatch. Every check runs on the host before the first
// launch, so a rejected call launches nothing and touches no device state.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "bsa.h"
#include "launch.h"

namespace {

thread_local char g_last_error[256] = "";

bsa_status fail(bsa_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
bsa_status fail(bsa_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

// Selection keeps a tile's score rows in 128 KB of LDS (one row at least).
constexpr int kMaxSelectKeyBlocks = 32768;
// The backward's transposed selection and per-row masks.
constexpr int kMaxBlocks = 4096;
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

struct Checked {
  bsa::Geom g;
  bool empty;
};

// Validates the problem and fills the kernel geometry.
bsa_status check_problem(const bsa_problem* p, Checked* out) {
  if (!p) return fail(BSA_ERR_INVALID_ARG, "problem is NULL");
  if (p->batch < 0 || p->heads < 0)
    return fail(BSA_ERR_INVALID_ARG, "batch and heads must be >= 0");
  if (p->T <= 0 || p->H <= 0 || p->W <= 0)
    return fail(BSA_ERR_INVALID_ARG, "latent grid T, H, W must be positive");
  if (p->ct <= 0 || p->ch <= 0 || p->cw <= 0)
    return fail(BSA_ERR_INVALID_ARG, "chunk extents must be positive");
  if (p->head_dim <= 0) return fail(BSA_ERR_INVALID_ARG, "head_dim must be positive");
  if (p->head_dim != bsa::kHeadDim)
    return fail(BSA_ERR_UNSUPPORTED, "head_dim %d: only 128 is implemented", p->head_dim);
  const long nq = (long)p->ct * p->ch * p->cw;
  if (nq != 64 && nq != bsa::kBlockTokens)
    return fail(BSA_ERR_UNSUPPORTED,
                "chunk %dx%dx%d: query blocks of 64 or 128 tokens are implemented", p->ct, p->ch,
                p->cw);
  if (p->cond_frames < 0 || p->cond_frames % p->ct || (p->cond_frames && p->cond_frames >= p->T))
    return fail(BSA_ERR_INVALID_ARG, "cond_frames %d must be a multiple of ct=%d and < T=%d",
                p->cond_frames, p->ct, p->T);
  if (!(p->scale == p->scale)) return fail(BSA_ERR_INVALID_ARG, "scale is NaN");
  const bool own_key_chunk = p->ctk != 0 || p->chk != 0 || p->cwk != 0;
  const int ctk = own_key_chunk ? p->ctk : p->ct;
  const int chk = own_key_chunk ? p->chk : p->ch;
  const int cwk = own_key_chunk ? p->cwk : p->cw;
  if (own_key_chunk) {
    if (ctk <= 0 || chk <= 0 || cwk <= 0)
      return fail(BSA_ERR_INVALID_ARG, "key chunk extents must all be positive (or all 0)");
    const long nk = (long)ctk * chk * cwk;
    if (nk != 64 && nk != 128 && nk != 256 && nk != 512 && nk != 1024)
      return fail(BSA_ERR_UNSUPPORTED,
                  "key chunk %dx%dx%d: key blocks of 64, 128, 256, 512 or 1024 tokens are "
                  "implemented", ctk, chk, cwk);
    if (p->cond_frames % ctk)
      return fail(BSA_ERR_INVALID_ARG, "cond_frames %d must be a multiple of ctk=%d",
                  p->cond_frames, ctk);
  }
  const long S = (long)p->T * p->H * p->W;
  // The attention kernel addresses one (batch, head) of K or V (S x 256 bytes)
  // through a buffer resource with a 32-bit size.
  if (S >= (1L << 24))
    return fail(BSA_ERR_UNSUPPORTED, "sequence of %ld tokens is too long (at most 2^24 - 1)", S);
  const long bh = (long)p->batch * p->heads;
  if (bh > (1L << 24)) return fail(BSA_ERR_UNSUPPORTED, "batch*heads = %ld is too large", bh);
  // Block counts are ceilings: a chunk that does not divide the grid leaves
  // partial blocks at its far edge.
  auto cdiv = [](long a, long b) { return (a + b - 1) / b; };
  const long nhw = cdiv(p->H, p->ch) * cdiv(p->W, p->cw);
  const long nb = cdiv(p->T, p->ct) * nhw;
  if ((unsigned long)nb * (unsigned long)nhw >= (1ul << 32))
    return fail(BSA_ERR_UNSUPPORTED, "block grid %ld x %ld is too large", nb, nhw);
  const long nhwk = cdiv(p->H, chk) * cdiv(p->W, cwk);
  const long nbk = cdiv(p->T, ctk) * nhwk;
  if ((unsigned long)nbk * (unsigned long)nhwk >= (1ul << 32))
    return fail(BSA_ERR_UNSUPPORTED, "key block grid %ld x %ld is too large", nbk, nhwk);
  bsa::Geom& g = out->g;
  g.bh = (int)bh;
  g.S = (int)S;
  g.T = p->T;
  g.H = p->H;
  g.W = p->W;
  g.ct = p->ct;
  g.ch = p->ch;
  g.cw = p->cw;
  g.nH = (int)cdiv(p->H, p->ch);
  g.nW = (int)cdiv(p->W, p->cw);
  g.nb = (int)nb;
  g.nq = (int)nq;
  g.cond_blocks = (p->cond_frames / p->ct) * g.nH * g.nW;
  g.scale = p->scale > 0.f ? p->scale : 1.0f / sqrtf((float)p->head_dim);
  g.ctk = ctk;
  g.chk = chk;
  g.cwk = cwk;
  g.nHk = (int)cdiv(p->H, chk);
  g.nWk = (int)cdiv(p->W, cwk);
  g.nk = ctk * chk * cwk;
  g.nbk = (int)nbk;
  g.cond_kblocks = (p->cond_frames / ctk) * g.nHk * g.nWk;
  g.partial = (p->T % p->ct || p->H % p->ch || p->W % p->cw || p->T % ctk || p->H % chk ||
               p->W % cwk)
                  ? 1
                  : 0;
  out->empty = (bh == 0);
  return BSA_OK;
}

bsa_status check_params(const bsa_select_params* sp) {
  if (!sp) return fail(BSA_ERR_INVALID_ARG, "select params are NULL");
  if (sp->mode == BSA_TOPK) {
    if (sp->k < 1) return fail(BSA_ERR_INVALID_ARG, "top-k needs k >= 1 (got %d)", sp->k);
  } else if (sp->mode == BSA_CDF) {
    if (!(sp->cdf_p > 0.f && sp->cdf_p <= 1.f))
      return fail(BSA_ERR_INVALID_ARG, "CDF threshold p must be in (0, 1]");
    if (sp->k_min < 1 || sp->k_max < sp->k_min)
      return fail(BSA_ERR_INVALID_ARG, "CDF needs 1 <= k_min <= k_max (got %d, %d)", sp->k_min,
                  sp->k_max);
  } else {
    return fail(BSA_ERR_INVALID_ARG, "unknown selection mode %d", sp->mode);
  }
  return BSA_OK;
}

// Selection workspace: pooled Q then pooled K (fp32); the pooled scores stay
// in LDS.
struct SelectLayout {
  size_t qp, kp, total;
};

SelectLayout select_layout(const bsa::Geom& g) {
  SelectLayout L;
  L.qp = 0;
  L.kp = align_up((size_t)g.bh * g.nb * bsa::kHeadDim * sizeof(float));
  L.total = L.kp + align_up((size_t)g.bh * g.nbk * bsa::kHeadDim * sizeof(float));
  return L;
}

size_t attention_ws(const bsa::Geom&) { return 0; }

// Launch status is read with hipGetLastError, which reports the last error
// of any HIP call on the thread. An error some earlier call left pending (the
// caller's own, or one a runtime fallback recorded without failing) is not
// this library's to report, so it is cleared before the library launches.
void clear_pending_error() { (void)hipGetLastError(); }

bsa_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess)
    return fail(BSA_ERR_LAUNCH, "%s launch failed: %s", what, hipGetErrorString(e));
  return BSA_OK;
}

bsa_status attention_common(const bsa_problem* problem, const void* q, const void* k,
                            const void* v, const int32_t* idx, const int32_t* cnt,
                            int32_t idx_stride, void* o, float* lse, void* workspace,
                            size_t workspace_bytes, void* stream, bool dense,
                            bool noisy_only = false) {
  Checked c;
  bsa_status st = check_problem(problem, &c);
  if (st != BSA_OK) return st;
  if (c.empty) return BSA_OK;
  if (!q || !k || !v || !o) return fail(BSA_ERR_INVALID_ARG, "q, k, v and o must be non-NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(BSA_ERR_INVALID_ARG, "q, k, v and o must be 16-byte aligned");
  if (!dense) {
    if (!idx || !cnt) return fail(BSA_ERR_INVALID_ARG, "idx and cnt must be non-NULL");
    if (idx_stride < 1) return fail(BSA_ERR_INVALID_ARG, "idx_stride must be >= 1");
  }
  if (o == q || o == k || o == v) return fail(BSA_ERR_INVALID_ARG, "o must not alias q, k or v");
  if (lse && ((uintptr_t)lse & 3u)) return fail(BSA_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  if (lse && ((const void*)lse == q || (const void*)lse == k || (const void*)lse == v ||
              (const void*)lse == o))
    return fail(BSA_ERR_INVALID_ARG, "lse must not alias q, k, v or o");
  const size_t need = attention_ws(c.g);
  if (workspace_bytes < need)
    return fail(BSA_ERR_WORKSPACE, "attention needs %zu workspace bytes (got %zu)", need,
                workspace_bytes);
  (void)workspace;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  clear_pending_error();
  return launched(bsa::launch_attention(c.g, static_cast<const bsa::bf16_bits*>(q),
                                        static_cast<const bsa::bf16_bits*>(k),
                                        static_cast<const bsa::bf16_bits*>(v), idx, cnt,
                                        dense ? 1 : idx_stride, dense,
                                        static_cast<bsa::bf16_bits*>(o), lse,
                                        noisy_only ? c.g.cond_blocks : 0, s),
                  "attention");
}

size_t cond_cache_bytes(const bsa::Geom& g) {
  return (size_t)g.bh * g.cond_kblocks * bsa::kHeadDim * sizeof(float);
}

// Selection for all query blocks, or (noisy) for the noisy ones only, with
// the condition key blocks' pooled keys taken from `cache`.
bsa_status select_common(const bsa_problem* problem, const bsa_select_params* params,
                         const void* q, const void* k, const float* cache, size_t cache_bytes,
                         int32_t* idx, int32_t* cnt, void* workspace, size_t workspace_bytes,
                         void* stream, bool noisy) {
  Checked c;
  bsa_status st = check_problem(problem, &c);
  if (st != BSA_OK) return st;
  st = check_params(params);
  if (st != BSA_OK) return st;
  if (c.empty) return BSA_OK;
  if (c.g.nbk > kMaxSelectKeyBlocks)
    return fail(BSA_ERR_UNSUPPORTED, "%d key blocks per head: selection supports at most %d",
                c.g.nbk, kMaxSelectKeyBlocks);
  if (!q || !k || !idx || !cnt)
    return fail(BSA_ERR_INVALID_ARG, "q, k, idx and cnt must be non-NULL");
  if (!aligned16(q) || !aligned16(k)) return fail(BSA_ERR_INVALID_ARG, "q and k must be 16-byte aligned");
  const int row0 = noisy ? c.g.cond_blocks : 0;
  const int kb0 = noisy ? c.g.cond_kblocks : 0;
  if (kb0 > 0) {
    if (!cache) return fail(BSA_ERR_INVALID_ARG, "the condition cache must be non-NULL");
    if (!aligned16(cache)) return fail(BSA_ERR_INVALID_ARG, "the condition cache must be 16-byte aligned");
    if (cache_bytes < cond_cache_bytes(c.g))
      return fail(BSA_ERR_WORKSPACE, "the condition cache needs %zu bytes (got %zu)",
                  cond_cache_bytes(c.g), cache_bytes);
  }
  const SelectLayout L = select_layout(c.g);
  if (!workspace || workspace_bytes < L.total)
    return fail(BSA_ERR_WORKSPACE, "select needs %zu workspace bytes (got %zu)", L.total,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned16(workspace)) return fail(BSA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  const int stride = params->mode == BSA_TOPK ? params->k : params->k_max;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  float* qp = reinterpret_cast<float*>(ws + L.qp);
  float* kp = reinterpret_cast<float*>(ws + L.kp);
  const bsa::bf16_bits* qb = static_cast<const bsa::bf16_bits*>(q);
  const bsa::bf16_bits* kb = static_cast<const bsa::bf16_bits*>(k);
  clear_pending_error();
  if (c.g.nq == bsa::kBlockTokens && c.g.nk == bsa::kBlockTokens && c.g.ctk == c.g.ct &&
      c.g.chk == c.g.ch && !c.g.partial) {
    st = launched(bsa::launch_pool(c.g, qb, kb, qp, kp, row0, s), "pool");
  } else {
    st = launched(bsa::launch_pool_queries(c.g, qb, qp, row0, s), "pool");
    if (st != BSA_OK) return st;
    st = launched(bsa::launch_pool_keys(c.g, kb, kp, kb0, c.g.nbk, c.g.nbk, s), "pool");
  }
  if (st != BSA_OK) return st;
  if (kb0 > 0) {
    // Cached condition rows into the leading rows of each head's pooled keys.
    const size_t row_bytes = (size_t)bsa::kHeadDim * sizeof(float);
    const hipError_t e = hipMemcpy2DAsync(kp, (size_t)c.g.nbk * row_bytes, cache, kb0 * row_bytes,
                                          kb0 * row_bytes, (size_t)c.g.bh, hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess)
      return fail(BSA_ERR_LAUNCH, "condition cache copy failed: %s", hipGetErrorString(e));
  }
  return launched(bsa::launch_select(c.g, qp, kp, params->mode, params->k, params->cdf_p,
                                     params->k_min, params->k_max, stride, idx, cnt, row0, s),
                  "select");
}

struct BwdLayout {
  size_t stats, mask, total;
  int nbw;
};

// Backward workspace: per (batch*head, query block) 128 values lse*log2(e)
// and 128 values D (fp32), then the key-block x query-block bit mask (nbk
// rows of ceil(nb/32) words per batch*head).
BwdLayout bwd_layout(const bsa::Geom& g) {
  BwdLayout L;
  L.nbw = (g.nb + 31) / 32;
  L.stats = 0;
  L.mask = align_up((size_t)g.bh * g.nb * 2 * bsa::kBlockTokens * sizeof(float));
  L.total = L.mask + align_up((size_t)g.bh * g.nbk * L.nbw * sizeof(uint32_t));
  return L;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

// Static device scratch for bsa_select_noalloc: every GPU the library runs on
// holds one copy until the process ends. In host code `scratch` names a
// host-side stand-in, never the device array: the device address comes from
// hipGetSymbolAddress, once per device, and only that address is used.
constexpr size_t kScratchBytes = size_t(64) << 20;
__device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
struct ScratchSlot {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};
ScratchSlot g_scratch[kMaxDevices];

// Device address of the current device's scratch array, looked up on the
// first call on that device (with that device current).
bsa_status scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(BSA_ERR_LAUNCH, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(BSA_ERR_UNSUPPORTED, "device %d: the static scratch serves devices 0..%d", dev,
                kMaxDevices - 1);
  ScratchSlot& slot = g_scratch[dev];
  std::call_once(slot.once, [&slot] {
    slot.err = hipGetSymbolAddress(&slot.ptr, HIP_SYMBOL(scratch));
  });
  if (slot.err != hipSuccess || !slot.ptr)
    return fail(BSA_ERR_LAUNCH, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                hipGetErrorString(slot.err));
  *out = slot.ptr;
  return BSA_OK;
}

}  // namespace

extern "C" {

int32_t bsa_index_stride(const bsa_problem* problem, const bsa_select_params* params) {
  if (problem) {
    Checked c;
    if (check_problem(problem, &c) != BSA_OK) return -1;
  }
  if (check_params(params) != BSA_OK) return -1;
  return params->mode == BSA_TOPK ? params->k : params->k_max;
}

size_t bsa_workspace_bytes(const bsa_problem* problem, const bsa_select_params* params) {
  Checked c;
  if (check_problem(problem, &c) != BSA_OK || check_params(params) != BSA_OK) return 0;
  const size_t sel = select_layout(c.g).total;
  const size_t att = attention_ws(c.g);
  return sel > att ? sel : att;
}

size_t bsa_select_workspace_bytes(const bsa_problem* problem, const bsa_select_params* params) {
  Checked c;
  if (check_problem(problem, &c) != BSA_OK || check_params(params) != BSA_OK) return 0;
  return select_layout(c.g).total;
}

size_t bsa_attention_workspace_bytes(const bsa_problem* problem) {
  Checked c;
  if (check_problem(problem, &c) != BSA_OK) return 0;
  return attention_ws(c.g);
}

bsa_status bsa_select(const bsa_problem* problem, const bsa_select_params* params,
                      const void* q, const void* k, int32_t* idx, int32_t* cnt,
                      void* workspace, size_t workspace_bytes, void* stream) {
  return select_common(problem, params, q, k, nullptr, 0, idx, cnt, workspace, workspace_bytes,
                       stream, false);
}

size_t bsa_select_noalloc_max_workspace_bytes(void) { return kScratchBytes; }

bsa_status bsa_select_noalloc(const bsa_problem* problem, const bsa_select_params* params,
                              const void* q, const void* k, int32_t* idx, int32_t* cnt,
                              void* stream) {
  Checked c;
  bsa_status st = check_problem(problem, &c);
  if (st != BSA_OK) return st;
  st = check_params(params);
  if (st != BSA_OK) return st;
  if (c.empty) return BSA_OK;
  const size_t need = select_layout(c.g).total;
  if (need > kScratchBytes)
    return fail(BSA_ERR_WORKSPACE,
                "select needs %zu workspace bytes; the static scratch of bsa_select_noalloc "
                "holds %zu (use bsa_select with a workspace)",
                need, kScratchBytes);
  void* ws = nullptr;
  st = scratch_for_current_device(&ws);
  if (st != BSA_OK) return st;
  return select_common(problem, params, q, k, nullptr, 0, idx, cnt, ws, kScratchBytes, stream,
                       false);
}

size_t bsa_cond_cache_bytes(const bsa_problem* problem) {
  Checked c;
  if (check_problem(problem, &c) != BSA_OK) return 0;
  return cond_cache_bytes(c.g);
}

bsa_status bsa_pool_cond_keys(const bsa_problem* problem, const void* k, float* cache,
                              size_t cache_bytes, void* stream) {
  Checked c;
  bsa_status st = check_problem(problem, &c);
  if (st != BSA_OK) return st;
  if (c.empty || c.g.cond_kblocks == 0) return BSA_OK;
  if (!k || !cache) return fail(BSA_ERR_INVALID_ARG, "k and cache must be non-NULL");
  if (!aligned16(k) || !aligned16(cache))
    return fail(BSA_ERR_INVALID_ARG, "k and cache must be 16-byte aligned");
  if (cache_bytes < cond_cache_bytes(c.g))
    return fail(BSA_ERR_WORKSPACE, "the condition cache needs %zu bytes (got %zu)",
                cond_cache_bytes(c.g), cache_bytes);
  clear_pending_error();
  return launched(bsa::launch_pool_keys(c.g, static_cast<const bsa::bf16_bits*>(k), cache, 0,
                                        c.g.cond_kblocks, c.g.cond_kblocks,
                                        reinterpret_cast<hipStream_t>(stream)),
                  "pool");
}

bsa_status bsa_select_noisy(const bsa_problem* problem, const bsa_select_params* params,
                            const void* q, const void* k, const float* cache, size_t cache_bytes,
                            int32_t* idx, int32_t* cnt, void* workspace, size_t workspace_bytes,
                            void* stream) {
  return select_common(problem, params, q, k, cache, cache_bytes, idx, cnt, workspace,
                       workspace_bytes, stream, true);
}

bsa_status bsa_attention(const bsa_problem* problem, const void* q, const void* k, const void* v,
                         const int32_t* idx, const int32_t* cnt, int32_t idx_stride, void* o,
                         void* workspace, size_t workspace_bytes, void* stream) {
  return attention_common(problem, q, k, v, idx, cnt, idx_stride, o, nullptr, workspace,
                          workspace_bytes, stream, false);
}

bsa_status bsa_attention_lse(const bsa_problem* problem, const void* q, const void* k,
                             const void* v, const int32_t* idx, const int32_t* cnt,
                             int32_t idx_stride, void* o, float* lse, void* workspace,
                             size_t workspace_bytes, void* stream) {
  if (problem && problem->batch > 0 && problem->heads > 0 && !lse)
    return fail(BSA_ERR_INVALID_ARG, "lse must be non-NULL");
  return attention_common(problem, q, k, v, idx, cnt, idx_stride, o, lse, workspace,
                          workspace_bytes, stream, false);
}

bsa_status bsa_attention_noisy(const bsa_problem* problem, const void* q, const void* k,
                               const void* v, const int32_t* idx, const int32_t* cnt,
                               int32_t idx_stride, void* o, void* workspace,
                               size_t workspace_bytes, void* stream) {
  return attention_common(problem, q, k, v, idx, cnt, idx_stride, o, nullptr, workspace,
                          workspace_bytes, stream, false, true);
}

size_t bsa_attention_bwd_workspace_bytes(const bsa_problem* problem) {
  Checked c;
  if (check_problem(problem, &c) != BSA_OK) return 0;
  return bwd_layout(c.g).total;
}

bsa_status bsa_attention_bwd(const bsa_problem* problem, const void* q, const void* k,
                             const void* v, const void* o, const void* dout, const float* lse,
                             const int32_t* idx, const int32_t* cnt, int32_t idx_stride, void* dq,
                             void* dk, void* dv, void* workspace, size_t workspace_bytes,
                             void* stream) {
  Checked c;
  bsa_status st = check_problem(problem, &c);
  if (st != BSA_OK) return st;
  if (c.empty) return BSA_OK;
  if (c.g.nb > kMaxBlocks)
    return fail(BSA_ERR_UNSUPPORTED, "%d blocks per head: the backward supports at most %d",
                c.g.nb, kMaxBlocks);
  if (c.g.nbk > kMaxBlocks)
    return fail(BSA_ERR_UNSUPPORTED, "%d key blocks per head: the backward supports at most %d",
                c.g.nbk, kMaxBlocks);
  const void* ins[6] = {q, k, v, o, dout, lse};
  void* outs[3] = {dq, dk, dv};
  for (const void* p : ins)
    if (!p) return fail(BSA_ERR_INVALID_ARG, "q, k, v, o, dout and lse must be non-NULL");
  for (void* p : outs)
    if (!p) return fail(BSA_ERR_INVALID_ARG, "dq, dk and dv must be non-NULL");
  if (!idx || !cnt) return fail(BSA_ERR_INVALID_ARG, "idx and cnt must be non-NULL");
  if (idx_stride < 1) return fail(BSA_ERR_INVALID_ARG, "idx_stride must be >= 1");
  for (int i = 0; i < 5; ++i)
    if (!aligned16(ins[i]))
      return fail(BSA_ERR_INVALID_ARG, "q, k, v, o and dout must be 16-byte aligned");
  for (void* p : outs)
    if (!aligned16(p)) return fail(BSA_ERR_INVALID_ARG, "dq, dk and dv must be 16-byte aligned");
  if ((uintptr_t)lse & 3u) return fail(BSA_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  const size_t tensor = (size_t)c.g.bh * c.g.S * bsa::kHeadDim * 2;
  const size_t sizes[6] = {tensor, tensor, tensor, tensor, tensor, (size_t)c.g.bh * c.g.S * 4};
  for (int a = 0; a < 3; ++a) {
    for (int b = 0; b < 6; ++b)
      if (overlaps(outs[a], tensor, ins[b], sizes[b]))
        return fail(BSA_ERR_INVALID_ARG, "dq, dk and dv must not overlap the inputs");
    for (int b = a + 1; b < 3; ++b)
      if (overlaps(outs[a], tensor, outs[b], tensor))
        return fail(BSA_ERR_INVALID_ARG, "dq, dk and dv must not overlap each other");
  }
  const BwdLayout L = bwd_layout(c.g);
  if (!workspace || workspace_bytes < L.total)
    return fail(BSA_ERR_WORKSPACE, "backward needs %zu workspace bytes (got %zu)", L.total,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned16(workspace)) return fail(BSA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  char* ws = static_cast<char*>(workspace);
  using bsa::bf16_bits;
  clear_pending_error();
  return launched(
      bsa::launch_attention_bwd(
          c.g, static_cast<const bf16_bits*>(q), static_cast<const bf16_bits*>(k),
          static_cast<const bf16_bits*>(v), static_cast<const bf16_bits*>(o),
          static_cast<const bf16_bits*>(dout), lse, idx, cnt, idx_stride,
          reinterpret_cast<float*>(ws + L.stats), reinterpret_cast<uint32_t*>(ws + L.mask),
          static_cast<bf16_bits*>(dq), static_cast<bf16_bits*>(dk), static_cast<bf16_bits*>(dv),
          reinterpret_cast<hipStream_t>(stream)),
      "attention backward");
}

bsa_status dense_attention(const bsa_problem* problem, const void* q, const void* k,
                           const void* v, void* o, void* workspace, size_t workspace_bytes,
                           void* stream) {
  return attention_common(problem, q, k, v, nullptr, nullptr, 1, o, nullptr, workspace,
                          workspace_bytes, stream, true);
}

const char* bsa_status_string(int32_t status) {
  switch (status) {
    case BSA_OK: return "ok";
    case BSA_ERR_INVALID_ARG: return "invalid argument";
    case BSA_ERR_UNSUPPORTED: return "unsupported problem";
    case BSA_ERR_WORKSPACE: return "workspace too small";
    case BSA_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

const char* bsa_last_error(void) { return g_last_error; }

}  // extern "C"
